// Device-side check of the preconditions the entry points cannot see from the
// host: the ragged offsets, the key positions a buffer row reads and the page
// ids behind them (page "generic_flare_mla_prefill_ragged_paged_plan", Args:
// input_row_offsets, cache_offsets and the row offsets; page
// "flare_mla_prefill", Args: valid_length, cache_row_offsets, cache_offsets).
//
// One wave per sequence.  Lane 0 checks the sequence's offsets; every lane
// then reads a share of the page-table entries of the positions the call would
// read (clamped to the sequence's page-table row, so the check itself reads
// only inside its arrays) and compares them with the page count.  Values are
// compared, never used as addresses.  Violations are ORed into one int32.
#include "check.h"

namespace mla {
namespace {

constexpr int CHECK_NT = 64;

__global__ void __launch_bounds__(CHECK_NT) check_kernel(CheckArgs a) {
  const uint32_t b = blockIdx.x;
  const uint32_t lane = threadIdx.x;
  uint32_t bits = 0;
  // the sequence's context length, when the new-token offsets are given
  uint64_t ctx = 0;
  bool ctx_known = false;
  if (a.valid_length) {
    const uint32_t q0 = a.valid_length[b], q1 = a.valid_length[b + 1];
    if (lane == 0) {
      if (b == 0 && q0 != 0) bits |= CHECK_Q_OFFSETS;
      if (q1 < q0) bits |= CHECK_Q_OFFSETS;
      if (a.tokens_known && b + 1 == a.batch && q1 != a.tokens) bits |= CHECK_Q_OFFSETS;
      if (a.q_max && q1 >= q0 && q1 - q0 > a.q_max) bits |= CHECK_Q_OFFSETS;
    }
    ctx = (uint64_t)a.cache_lengths[b] + (q1 >= q0 ? q1 - q0 : 0u);
    ctx_known = true;
  }
  // positions [lo, hi) the call reads for this sequence
  uint64_t lo = 0, hi = ctx;
  if (a.row_offsets) {
    const uint32_t r0 = a.row_offsets[b], r1 = a.row_offsets[b + 1];
    const uint32_t len = r1 >= r0 ? r1 - r0 : 0u;
    if (lane == 0) {
      if (r1 < r0) bits |= CHECK_ROW_OFFSETS;
      if (a.row_capacity && b + 1 == a.batch && r1 > a.row_capacity) bits |= CHECK_ROW_OFFSETS;
    }
    lo = a.row_positions ? a.row_positions[b] : 0u;
    hi = lo + len;
    if (lane == 0 && ctx_known && hi > ctx) bits |= CHECK_POSITIONS;
  }
  if (a.page_table && hi > lo) {
    const uint64_t limit = (uint64_t)a.max_pages * a.page_size;
    if (lane == 0 && hi > limit) bits |= CHECK_POSITIONS;
    const uint64_t last = (hi < limit ? hi : limit) - 1;
    if (lo <= last) {
      const uint32_t* pt = a.page_table + (size_t)b * a.max_pages;
      for (uint64_t pg = lo / a.page_size + lane; pg <= last / a.page_size; pg += CHECK_NT)
        if (pt[pg] >= a.num_pages) bits |= CHECK_PAGE_IDS;
    }
  }
  if (bits) atomicOr(a.violations, (int)bits);
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(check_kernel, dim3(a.batch), dim3(CHECK_NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
