// Device-side helpers shared by the gfx950 kernels of the MLA prefill library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

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

constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float LN2_F = 0.6931471805599453f;

// Combine weights of two partial softmax results from their log-sum-exps
// (natural log): the union's lse is ln(e^la + e^lb) and each side weighs
// e^(l_x - lse).  Both sides empty (-inf) gives weights 0 and lse -inf; one side
// empty passes the other through exactly (weight 1, its lse unchanged).
struct MergeWeights {
  float wa, wb, lse;
};
__device__ __forceinline__ MergeWeights merge_weights(float la, float lb) {
  const float mm = fmaxf(la, lb);
  if (mm == -INFINITY) return MergeWeights{0.f, 0.f, -INFINITY};
  const float ea = __builtin_amdgcn_exp2f((la - mm) * LOG2E_F);
  const float eb = __builtin_amdgcn_exp2f((lb - mm) * LOG2E_F);
  const float sum = ea + eb;                       // in [1, 2]
  return MergeWeights{ea / sum, eb / sum, mm + __builtin_amdgcn_logf(sum) * LN2_F};
}

// Where a unit's finished rows go: the output (bf16 or fp32), optionally the
// log-sum-exp, optionally merged with an earlier partial.
struct RowTarget {
  void* out;
  uint32_t out_fp32;
  float* lse;
  const float* prev;
  const float* prev_lse;
};

// Target of one unit.  A plain call takes its own arguments.  In row mode (one
// row of a plan that cut the contexts over several buffer rows, rows run in
// order): sequence b's first row (its slice starts at cache position 0) starts
// the fp32 partial in acc / acc_lse, a middle row merges into it in place, and
// the last row (its slice ends at the context's end, p_b + n_b) merges and writes
// the output; a sequence whose context one row holds writes the output directly.
__device__ __forceinline__ RowTarget row_target(const PrefillArgs& a, bool first, bool last) {
  if (!a.row_mode) return RowTarget{a.out, a.out_fp32, a.lse, a.prev_out, a.prev_lse};
  if (first && last) return RowTarget{a.out, a.out_fp32, a.lse, nullptr, nullptr};
  if (first) return RowTarget{a.acc, 1u, a.acc_lse, nullptr, nullptr};
  if (!last) return RowTarget{a.acc, 1u, a.acc_lse, a.acc, a.acc_lse};
  return RowTarget{a.out, a.out_fp32, a.lse, a.acc, a.acc_lse};
}

// Stores one lane's share of a finished query row (row = token * H + head).
// o[d][4g + k] is output column 32d + 8g + 4hf + k before normalisation, `inv`
// normalises it, and lse2 is the row's log-sum-exp in log2 units (-inf when the
// call saw no key for the row).  With an earlier partial in t.prev / t.prev_lse
// the two are combined by merge_weights; the earlier side is read only where
// its weight is non-zero.  The output is written as bf16 (rounded to
// nearest-even) or fp32, and the lower half's lanes store the log-sum-exp, in
// natural-log units, when t.lse is set.  Each lane reads the earlier partial's
// elements before it writes them, so out / lse may be the same buffers as
// prev / prev_lse.
// PLAIN: bf16 output, no log-sum-exp, no earlier partial (only t.out is read).
template <bool PLAIN>
__device__ __forceinline__ void store_output_row(const RowTarget& t, size_t row, int hf, const f32x16 (&o)[4],
                                                 float inv, float lse2) {
  if constexpr (PLAIN) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dv = d * 32 + g * 8 + hf * 4;
        const uint32_t w0 = pack_bf16x2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(t.out) + row * 128 + dv) = u32x2{w0, w1};
      }
    }
    return;
  }
  float w_self = inv, w_prev = 0.f;
  float lse = lse2 * LN2_F;
  const float* prev = nullptr;
  if (t.prev) {
    const MergeWeights mw = merge_weights(t.prev_lse[row], lse);
    w_self = inv * mw.wb;
    w_prev = mw.wa;
    lse = mw.lse;
    if (w_prev > 0.f) prev = t.prev + row * 128;
  }
  if (t.lse && hf == 0) t.lse[row] = lse;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dv = d * 32 + g * 8 + hf * 4;
      f32x4 val = {o[d][4 * g] * w_self, o[d][4 * g + 1] * w_self, o[d][4 * g + 2] * w_self,
                   o[d][4 * g + 3] * w_self};
      if (prev) {
        const f32x4 pv = *reinterpret_cast<const f32x4*>(prev + dv);
        val = {__builtin_fmaf(w_prev, pv[0], val[0]), __builtin_fmaf(w_prev, pv[1], val[1]),
               __builtin_fmaf(w_prev, pv[2], val[2]), __builtin_fmaf(w_prev, pv[3], val[3])};
      }
      if (t.out_fp32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(t.out) + row * 128 + dv) = val;
      } else {
        const uint32_t w0 = pack_bf16x2(val[0], val[1]);
        const uint32_t w1 = pack_bf16x2(val[2], val[3]);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(t.out) + row * 128 + dv) = u32x2{w0, w1};
      }
    }
  }
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
// groups of 8, so the 8 consecutive ids that reach the 4 shader engines (two
// each) are the same (sequence, tile) of 8 heads and cost the same (tiles past
// a short sequence's end then fall evenly on all engines too; groups of 8
// measured 2-3 % faster than groups of 4 on a 4-sequence batch, equal on 8 and
// 16 sequences, and groups of 16 up to 4 % slower).  With one sequence, neighbouring
// tiles of one head already cost nearly the same and one head at a time keeps
// the XCD's L2 on one K/V stream.  Other head counts: tiles longest-first, then
// sequence, then head, over the whole chip.
__device__ __forceinline__ bool decode_unit(uint32_t bid, uint32_t H, uint32_t B, uint32_t Q, WorkUnit& u) {
  if (bid >= H * B * Q) return false;
  if ((H & 7u) == 0) {
    const uint32_t hx = H >> 3, xcd = bid & 7u, j = bid >> 3;
    const uint32_t g = B > 1 ? 8u : 1u;
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

// Key split, for grids with too few units to keep every CU busy until the end
// (a few sequences at a few heads, where one long query tile outlasts the rest
// of the grid): a query tile whose visible key range [0, jend) holds more than
// split_keys keys is computed by two units, one per half of its key tiles, each
// writing a normalised fp32 partial and its log-sum-exp to the workspace; a
// second pass merges the two.  The attention kernels and the merge pass take
// the decision from these same values.
__device__ __forceinline__ bool kv_split_tile(int32_t jend, uint32_t split_keys) {
  return split_keys != 0u && jend > (int32_t)split_keys;
}

// Workspace target of half c (0: first key tiles, 1: the rest) of a split tile:
// partial rows at ws + c*T*H*128, their log-sum-exp at ws + 2*T*H*128 + c*T*H.
__device__ __forceinline__ RowTarget kv_split_target(const PrefillArgs& a, uint32_t c) {
  const size_t plane = (size_t)a.tokens * a.heads;
  return RowTarget{a.ws + c * plane * 128, 1u, a.ws + 2 * plane * 128 + c * plane, nullptr, nullptr};
}

}  // namespace mla
