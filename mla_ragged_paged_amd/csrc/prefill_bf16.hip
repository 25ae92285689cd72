// Ragged, causally masked MLA prefill over a paged K_rope cache -- bf16 inputs,
// bf16 output, fp32 accumulation.  Semantics: page "flare_mla_prefill"
// (description and Args) with the paged k_rope operand; argument meanings of
// page "mla_prefill_v2_ragged" (Args).
//
// Work unit = (head h, sequence b, query tile of BM = 128 rows).  A workgroup of
// four waves owns one unit; wave w owns queries [32w, 32w+32) of the tile.
// Keys stream through LDS in tiles of BN = 64: K (128 nope columns from k_nope
// plus the 64 shared K_rope columns read through the page table) and V, both
// row-major, with the next tile's global loads in flight while the current one
// is consumed.
//
// Per wave and key tile, on the 32x32x16 bf16 MFMA:
//   S^T = K . Q^T  (A = K rows from LDS, B = the wave's Q held in registers),
//        so each lane owns one query column and 32 of the tile's 64 keys:
//        row max / sum need one exchange between the wave's two 32-lane halves;
//   online softmax in the exp2 domain (scale * log2 e folded in), masking only
//        on tiles that straddle the causal diagonal or the ragged tail;
//   O^T += V^T . P^T (A = V read transposed out of row-major LDS with
//        ds_read_b64_tr_b16, B = P^T straight from the S^T registers after a
//        bf16 rounding).  The 16 keys of one MFMA step are taken in the order
//        the S^T accumulator holds them; V is read in that same order.
#include "device_common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int BM = 128;            // queries per workgroup
constexpr int BN = 64;             // keys per tile
constexpr int NT = 256;            // threads per workgroup
constexpr int DQK = 192, DNOPE = 128, DROPE = 64, DV = 128;
constexpr int KS = DQK + 8;        // LDS row stride of K (bf16 elements)
constexpr int VS = DV + 32;        // LDS row stride of V (bf16 elements)

struct Tile {                      // one thread's share of a K/V tile, in flight
  i32x4 kn[4];
  i32x4 kr[2];
  i32x4 v[4];
};

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

__global__ void __launch_bounds__(NT, 2) prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN * VS];

  // ---- work unit: XCD-aware decode.  Workgroup ids go round-robin over the 8
  // XCDs, so id % 8 picks a contiguous range of the (head, sequence, tile)
  // order; each XCD's L2 then serves whole heads.  Tiles of a sequence run
  // longest-first.
  const uint32_t bid = blockIdx.x;
  const uint32_t logical = (bid & 7u) * a.units_per_xcd + (bid >> 3);
  if (logical >= a.units) return;
  const uint32_t qt = a.qtiles - 1u - logical % a.qtiles;
  const uint32_t hb = logical / a.qtiles;
  const uint32_t b = hb % a.batch;
  const uint32_t h = hb / a.batch;
  const uint32_t t0 = a.valid_length[b];
  const uint32_t n = a.valid_length[b + 1] - t0;
  const uint32_t i0 = qt * BM;
  if (i0 >= n) return;

  const uint32_t H = a.heads;
  const uint32_t p = a.cache_lengths[b];
  const uint32_t g0 = a.cache_row_offsets[b];
  const uint32_t len = a.cache_row_offsets[b + 1] - g0;
  const uint32_t c0 = a.cache_offsets ? a.cache_offsets[b] : 0u;
  const uint32_t i_last = min(n, i0 + BM) - 1u;
  // keys some query of the tile can see: c0 + j <= p + i_last
  const int64_t jlim = (int64_t)p + i_last - c0 + 1;
  const uint32_t jend = jlim <= 0 ? 0u : (uint32_t)min<int64_t>(jlim, len);
  const uint32_t nkt = (jend + BN - 1) / BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, hf = lane >> 5;
  const uint32_t iw0 = i0 + 32u * w;                 // wave's first query
  const bool wave_rows = iw0 < n;
  const uint32_t my_i = iw0 + li;                    // this lane's query column
  const bool row_valid = my_i < n;
  const int64_t my_qpos = (int64_t)p + my_i;
  const int64_t wq_first = (int64_t)p + iw0;
  const int64_t wq_last = (int64_t)p + min(n, iw0 + 32u) - 1;

  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ KN = static_cast<const uint16_t*>(a.k_nope);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const uint16_t* __restrict__ CR = static_cast<const uint16_t*>(a.cache);
  const uint32_t* __restrict__ PT = a.page_table + (size_t)b * a.max_pages;

  // ---- Q^T operands: lane (li, hf) holds q[t][h][16ks + 8hf .. +7] for its query
  bf16x8 qop[12];
  {
    const uint32_t qi = row_valid ? my_i : 0u;
    const uint16_t* qrow = Q + ((size_t)(t0 + qi) * H + h) * DQK + hf * 8;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      i32x4 x = ld16(qrow + ks * 16);
      if (!row_valid) x = i32x4{0, 0, 0, 0};
      qop[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  auto load_tile = [&](uint32_t kt, Tile& tl) {
    const uint32_t j0 = kt * BN;
#pragma unroll
    for (int u = 0; u < 4; ++u) {                    // nope and V: 64 rows x 16 chunks
      const int c = tid + NT * u;
      const uint32_t j = j0 + (c >> 4);
      const int col = (c & 15) * 8;
      i32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
      if (j < jend) {
        const size_t off = ((size_t)(g0 + j) * H + h) * DNOPE + col;
        kx = ld16(KN + off);
        vx = ld16(V + off);
      }
      tl.kn[u] = kx;
      tl.v[u] = vx;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {                    // rope: 64 rows x 8 chunks
      const int c = tid + NT * u;
      const uint32_t j = j0 + (c >> 3);
      const int col = (c & 7) * 8;
      i32x4 rx = {0, 0, 0, 0};
      if (j < jend) {
        const uint32_t pos = c0 + j;
        uint32_t page, slot;
        if (a.page_shift < 32u) { page = PT[pos >> a.page_shift]; slot = pos & (a.page_size - 1u); }
        else { page = PT[pos / a.page_size]; slot = pos % a.page_size; }
        rx = ld16(CR + ((size_t)page * a.page_size + slot) * a.row_width + a.rope_col + col);
      }
      tl.kr[u] = rx;
    }
  };
  auto store_tile = [&](const Tile& tl) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + NT * u;
      const int row = c >> 4, col = (c & 15) * 8;
      *reinterpret_cast<i32x4*>(&Ks[row * KS + col]) = tl.kn[u];
      *reinterpret_cast<i32x4*>(&Vs[row * VS + col]) = tl.v[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + NT * u;
      const int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<i32x4*>(&Ks[row * KS + DNOPE + col]) = tl.kr[u];
    }
  };

  // ---- running softmax state (exp2 domain) and output accumulator O^T
  const float c_log2 = a.scale * 1.4426950408889634f;
  float m_run = -1e30f;                              // finite: exp2(m_old - m_new) stays defined
  float l_run = 0.f;                                 // this lane's share of the row sum
  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x16{};

  // transposed-read source address of this lane inside a 16-key MFMA step
  // (see ds_read_b64_tr_b16: lane 16g+4e+c supplies row e, columns 4c..4c+3)
  const int tr_g = lane >> 4, tr_e = (lane >> 2) & 3, tr_c = lane & 3;
  const int tr_row = 4 * (tr_g >> 1) + tr_e;         // key within the step (+8 for the second read)
  const int tr_col = (tr_g & 1) * 16 + 4 * tr_c;     // dv within a 32-wide block

  Tile tl;
  if (nkt > 0) {
    load_tile(0, tl);
    store_tile(tl);
  }
  __syncthreads();

  for (uint32_t kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) load_tile(kt + 1, tl);
    const uint32_t j0 = kt * BN;
    const int64_t kfirst = (int64_t)c0 + j0;
    if (wave_rows && kfirst <= wq_last) {
      const bool full = (j0 + BN <= len) && (kfirst + BN - 1 <= wq_first);
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + li) * KS + ks * 16 + hf * 8]);
          s[kb] = mfma_bf16(ka, qop[ks], s[kb]);
        }
      }
      // scale, mask, row max.  s[kb][r] is key j0 + 32kb + 8(r/4) + 4hf + r%4.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][r] * c_log2;
          if (!full) {
            const uint32_t j = j0 + kb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
            const bool vis = (j < len) && ((int64_t)c0 + j <= my_qpos);
            x = vis ? x : -INFINITY;
          }
          s[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = max_across_halves(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(s[kb][r] - m_new);
          s[kb][r] = e;
          psum += e;
        }
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] *= alpha;

      // O^T += V^T P^T, four 16-key steps
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int kb = kk >> 1, sub = kk & 1;
        uint32_t pw[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) pw[x] = pack_bf16x2(s[kb][8 * sub + 2 * x], s[kb][8 * sub + 2 * x + 1]);
        const bf16x8 pop = __builtin_bit_cast(bf16x8, i32x4{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]});
        const int key = kk * 16 + tr_row;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint16_t* base = &Vs[key * VS + d * 32 + tr_col];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(base));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(base + 8 * VS));
          const bf16x8 va = __builtin_bit_cast(bf16x8, i32x4{__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                                                             __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]});
          o[d] = mfma_bf16(va, pop, o[d]);
        }
      }
    }
    __syncthreads();
    if (kt + 1 < nkt) {
      store_tile(tl);
      __syncthreads();
    }
  }

  // ---- epilogue: combine the two halves' row sums, normalise, round to bf16
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_valid) {
    uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)(t0 + my_i) * H + h) * DV;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dv = d * 32 + g * 8 + hf * 4;
        const uint32_t w0 = pack_bf16x2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + dv) = u32x2{w0, w1};
      }
    }
  }
}

hipError_t launch_prefill_bf16(PrefillArgs a, uint32_t q_max, hipStream_t stream) {
  a.qtiles = (q_max + BM - 1) / BM;
  const uint64_t units = (uint64_t)a.heads * a.batch * a.qtiles;
  a.units = (uint32_t)units;
  const uint64_t grid = (units + 7) / 8 * 8;
  a.units_per_xcd = (uint32_t)(grid / 8);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((uint32_t)grid), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
