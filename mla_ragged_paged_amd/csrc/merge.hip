// Log-sum-exp combine of two partial attention results over disjoint key sets.
// When the plan of page "generic_flare_mla_prefill_ragged_paged_plan"
// (description, Args) cuts a sequence's context over several buffer rows, each
// row's attention is a softmax over part of the keys; two such partials, each a
// normalised output row and the log-sum-exp of its scores, combine into the
// softmax over the union.  The same combine is the second pass of the key
// split (kv_split_merge_kernel), which joins the two halves of a long query
// tile's keys computed by two workgroups.
//
// Elementwise and bound by HBM traffic: 32 lanes per (token, head) row, four
// fp32 columns (16 bytes) per lane, both lse values of the row read once per
// 32-lane group.
#include "device_common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int MERGE_NT = 256;
constexpr uint32_t SPLIT_BM = 128;   // queries per tile of the attention kernels

// One lane's four columns of a merged row: side a and side b (normalised fp32
// rows with their log-sum-exp) combine by merge_weights; a side with zero weight
// is not read (an empty partial's output is never used).  The lane at column 0
// writes the row's log-sum-exp when lse is set.
__device__ __forceinline__ void merge_row(void* out, uint32_t out_fp32, float* lse, const float* o_a,
                                          const float* lse_a, const float* o_b, const float* lse_b, size_t row,
                                          int col) {
  const MergeWeights mw = merge_weights(lse_a[row], lse_b[row]);
  f32x4 val = {0.f, 0.f, 0.f, 0.f};
  if (mw.wa > 0.f) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(o_a + row * 128 + col);
    val = {mw.wa * x[0], mw.wa * x[1], mw.wa * x[2], mw.wa * x[3]};
  }
  if (mw.wb > 0.f) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(o_b + row * 128 + col);
    val = {__builtin_fmaf(mw.wb, x[0], val[0]), __builtin_fmaf(mw.wb, x[1], val[1]),
           __builtin_fmaf(mw.wb, x[2], val[2]), __builtin_fmaf(mw.wb, x[3], val[3])};
  }
  if (lse && col == 0) lse[row] = mw.lse;
  if (out_fp32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + row * 128 + col) = val;
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + row * 128 + col) =
        u32x2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
  }
}

__global__ void __launch_bounds__(MERGE_NT) merge_kernel(MergeArgs a) {
  const uint64_t gid = (uint64_t)blockIdx.x * MERGE_NT + threadIdx.x;
  const uint64_t row = gid >> 5;
  if (row >= a.rows) return;
  merge_row(a.out, a.out_fp32, a.lse, a.o_a, a.lse_a, a.o_b, a.lse_b, row, (int)(gid & 31u) * 4);
}

// Second pass of the key split: one workgroup per (sequence, 128-query tile,
// head) of the attention grid; a tile the attention pass did not split returns
// at once, a split one merges its two halves' partial rows into the output
// (and log-sum-exp).  Its visible key range is computed as the attention
// kernels compute it, so both passes select the same tiles.  Lane l of the
// workgroup takes columns 4(l % 32) .. +3 of the tile's rows l / 32 + 8k,
// k < 16; every row's loads are issued before the first is used, so the pass
// waits for memory about twice rather than once per row.
__global__ void __launch_bounds__(MERGE_NT) kv_split_merge_kernel(PrefillArgs a) {
  const uint32_t H = a.heads;
  const uint32_t h = blockIdx.x % H, bq = blockIdx.x / H;
  const uint32_t b = bq / a.qtiles, qt = bq - b * a.qtiles;
  const uint32_t t0 = a.valid_length[b];
  const uint32_t n = a.valid_length[b + 1] - t0;
  const uint32_t i0 = qt * SPLIT_BM;
  if (i0 >= n) return;
  const int32_t p = (int32_t)a.cache_lengths[b];
  const int32_t len = (int32_t)(a.cache_row_offsets[b + 1] - a.cache_row_offsets[b]);
  const int32_t c0 = a.cache_offsets ? (int32_t)a.cache_offsets[b] : 0;
  const int32_t i_last = (int32_t)min(n, i0 + SPLIT_BM) - 1;
  const int32_t jend = a.causal ? max(0, min(p + i_last - c0 + 1, len)) : len;
  if (!kv_split_tile(jend, a.split_keys)) return;
  const RowTarget first = kv_split_target(a, 0), second = kv_split_target(a, 1);
  const float* o_a = static_cast<const float*>(first.out);
  const float* o_b = static_cast<const float*>(second.out);
  const int col = (int)(threadIdx.x & 31u) * 4;
  constexpr int ROWS = SPLIT_BM / (MERGE_NT / 32);
  size_t row[ROWS];
  bool live[ROWS];
  float la[ROWS], lb[ROWS];
#pragma unroll
  for (int k = 0; k < ROWS; ++k) {
    const int32_t i = (int32_t)i0 + (int32_t)(threadIdx.x >> 5) + k * (MERGE_NT / 32);
    live[k] = i <= i_last;
    row[k] = (size_t)(t0 + (uint32_t)min(i, i_last)) * H + h;
    la[k] = first.lse[row[k]];
    lb[k] = second.lse[row[k]];
  }
  MergeWeights mw[ROWS];
  f32x4 xa[ROWS], xb[ROWS];
#pragma unroll
  for (int k = 0; k < ROWS; ++k) {
    // a side with zero weight is not read (an empty partial's output is never used)
    mw[k] = merge_weights(la[k], lb[k]);
    xa[k] = mw[k].wa > 0.f ? *reinterpret_cast<const f32x4*>(o_a + row[k] * 128 + col) : f32x4{0.f, 0.f, 0.f, 0.f};
    xb[k] = mw[k].wb > 0.f ? *reinterpret_cast<const f32x4*>(o_b + row[k] * 128 + col) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int k = 0; k < ROWS; ++k) {
    if (!live[k]) continue;
    f32x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) val[e] = __builtin_fmaf(mw[k].wb, xb[k][e], mw[k].wa * xa[k][e]);
    if (a.lse && col == 0) a.lse[row[k]] = mw[k].lse;
    if (a.out_fp32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row[k] * 128 + col) = val;
    } else {
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row[k] * 128 + col) =
          u32x2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
    }
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const uint64_t blocks = (a.rows * 32 + MERGE_NT - 1) / MERGE_NT;
  hipLaunchKernelGGL(merge_kernel, dim3((uint32_t)blocks), dim3(MERGE_NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kv_split_merge(const PrefillArgs& a, hipStream_t stream) {
  const uint64_t blocks = (uint64_t)a.heads * a.batch * a.qtiles;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_split_merge_kernel, dim3((uint32_t)blocks), dim3(MERGE_NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
