// Log-sum-exp combine of two partial attention results over disjoint key sets.
// When the plan of page "generic_flare_mla_prefill_ragged_paged_plan"
// (description, Args) cuts a sequence's context over several buffer rows, each
// row's attention is a softmax over part of the keys; two such partials, each a
// normalised output row and the log-sum-exp of its scores, combine into the
// softmax over the union.
//
// Elementwise and bound by HBM traffic: 32 lanes per (token, head) row, four
// fp32 columns (16 bytes) per lane, both lse values of the row read once per
// 32-lane group.
#include "device_common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int MERGE_NT = 256;

__global__ void __launch_bounds__(MERGE_NT) merge_kernel(MergeArgs a) {
  const uint64_t gid = (uint64_t)blockIdx.x * MERGE_NT + threadIdx.x;
  const uint64_t row = gid >> 5;
  if (row >= a.rows) return;
  const int col = (int)(gid & 31u) * 4;
  const MergeWeights mw = merge_weights(a.lse_a[row], a.lse_b[row]);
  f32x4 val = {0.f, 0.f, 0.f, 0.f};
  // a side with zero weight is not read (an empty partial's output is never used)
  if (mw.wa > 0.f) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.o_a + row * 128 + col);
    val = {mw.wa * x[0], mw.wa * x[1], mw.wa * x[2], mw.wa * x[3]};
  }
  if (mw.wb > 0.f) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.o_b + row * 128 + col);
    val = {__builtin_fmaf(mw.wb, x[0], val[0]), __builtin_fmaf(mw.wb, x[1], val[1]),
           __builtin_fmaf(mw.wb, x[2], val[2]), __builtin_fmaf(mw.wb, x[3], val[3])};
  }
  if (a.lse && (gid & 31u) == 0) a.lse[row] = mw.lse;
  if (a.out_fp32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * 128 + col) = val;
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * 128 + col) =
        u32x2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const uint64_t blocks = (a.rows * 32 + MERGE_NT - 1) / MERGE_NT;
  hipLaunchKernelGGL(merge_kernel, dim3((uint32_t)blocks), dim3(MERGE_NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
