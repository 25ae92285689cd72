// Device-side helpers shared by the gfx950 kernels of the MLA prefill library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

#define MLA_LDS __attribute__((address_space(3)))

// 16-byte global load / store (the addresses used are 16-byte aligned).
__device__ __forceinline__ i32x4 ld16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }
__device__ __forceinline__ void st16(void* p, i32x4 v) { *reinterpret_cast<i32x4*>(p) = v; }

// Round two floats to bf16 (nearest-even) and pack them, low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Value of `x` from lane (l ^ 32): the two 32-lane halves of a wave swap.
__device__ __forceinline__ float swap_halves(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0..31 receive the upper half's value in r[1], lanes 32..63 the lower half's in r[0]
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float max_across_halves(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One work unit of the prefill kernels: (head, sequence, 128-query tile).
struct WorkUnit {
  uint32_t h, b, qt;
};

// Maps a workgroup id to its work unit; false for ids past the last unit.
// Workgroup ids go round-robin over the 8 XCDs (id % 8), and within an XCD
// round-robin over its 4 shader engines ((id / 8) % 4), each of which starts
// its workgroups in id order.  When H is a multiple of 8, XCD x takes heads
// [x*H/8, (x+1)*H/8), so its L2 serves those heads' K/V.  Within an XCD a
// sequence's tiles run longest-first; with several sequences the heads go in
// quads, so the 4 consecutive ids that reach the 4 shader engines are the same
// (sequence, tile) of 4 heads and cost the same (tiles past a short sequence's
// end then fall evenly on all engines too).  With one sequence, neighbouring
// tiles of one head already cost nearly the same and one head at a time keeps
// the XCD's L2 on one K/V stream.  Other head counts: tiles longest-first, then
// sequence, then head, over the whole chip.
__device__ __forceinline__ bool decode_unit(uint32_t bid, uint32_t H, uint32_t B, uint32_t Q, WorkUnit& u) {
  if (bid >= H * B * Q) return false;
  if ((H & 7u) == 0) {
    const uint32_t hx = H >> 3, xcd = bid & 7u, j = bid >> 3;
    const uint32_t g = B > 1 ? 4u : 1u;
    const uint32_t hs = j / (g * B * Q) * g;      // first head (within the XCD) of this group
    const uint32_t gl = min(g, hx - hs);          // heads in this group
    const uint32_t r = j - hs * B * Q;
    const uint32_t bq = r / gl;
    u.h = xcd * hx + hs + r % gl;
    u.b = bq / Q;
    u.qt = Q - 1u - bq % Q;
  } else {
    const uint32_t rest = bid / H;
    u.h = bid % H;
    u.b = rest % B;
    u.qt = Q - 1u - rest / B;
  }
  return true;
}

}  // namespace mla
