// Plan and gather kernels: page "generic_flare_mla_prefill_ragged_paged_plan"
// (Modular MAX API docs), description and Args.
//
// plan:   the batch's contexts (cached prefix + new tokens of every sequence, in
//         batch order) are cut into rows of `cap` tokens; each row records where
//         each sequence's slice starts in the row and in the sequence's cache.
// gather: copies one row's slices out of the paged cache into a contiguous buffer.
#include "device_common.h"
#include "kernels.h"

namespace mla {

// Every block rebuilds the batch's context prefix sums S[0..B] in LDS (B is at
// most MLA_MAX_BATCH) and then writes the plan rows assigned to it.
__global__ void __launch_bounds__(256) plan_kernel(PlanArgs a) {
  extern __shared__ uint64_t S[];             // [B + 1] context prefix sums
  __shared__ uint64_t part[4];                // per-wave totals
  const uint32_t tid = threadIdx.x;
  const uint32_t B = a.batch;
  const uint32_t per = (B + 255u) / 256u;
  const uint32_t b0 = min(B, tid * per), b1 = min(B, b0 + per);
  uint64_t sum = 0;
  for (uint32_t b = b0; b < b1; ++b) {
    const uint64_t L = (uint64_t)a.cache_lengths[b] + (uint64_t)(a.input_row_offsets[b + 1] - a.input_row_offsets[b]);
    S[b + 1] = L;
    sum += L;
  }
  // exclusive prefix of the 256 threads' sums: inclusive scan within each wave
  // (64-bit values moved as two 32-bit shuffles), then the waves' totals
  const int lane = (int)(tid & 63u), wv = (int)(tid >> 6);
  uint64_t incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)incl, (unsigned)d, 64);
    const uint32_t hi = __shfl_up((uint32_t)(incl >> 32), (unsigned)d, 64);
    if (lane >= d) incl += ((uint64_t)hi << 32) | lo;
  }
  if (lane == 63) part[wv] = incl;
  if (tid == 0) S[0] = 0;
  __syncthreads();
  uint64_t acc = incl - sum;
  for (int i = 0; i < wv; ++i) acc += part[i];
  for (uint32_t b = b0; b < b1; ++b) { acc += S[b + 1]; S[b + 1] = acc; }
  __syncthreads();

  const int64_t total = (int64_t)S[B];
  const int64_t cap = a.cap;
  const int64_t rows_needed = (total + cap - 1) / cap;
  if (blockIdx.x == 0 && tid == 0 && a.status) *a.status = rows_needed > (int64_t)a.rows ? 1 : 0;

  const uint32_t r_begin = blockIdx.x * a.rows_per_block;
  const uint32_t r_end = min(a.rows, r_begin + a.rows_per_block);
  for (uint32_t r = r_begin; r < r_end; ++r) {
    const int64_t lo = (int64_t)r * cap;
    const bool used = (int64_t)r < rows_needed;
    uint32_t* bro = a.buffer_row_offsets + (size_t)r * (B + 1);
    uint32_t* co = a.cache_offsets + (size_t)r * B;
    for (uint32_t b = tid; b <= B; b += 256) {
      const int64_t x = (int64_t)S[b] - lo;
      bro[b] = used ? (uint32_t)(x < 0 ? 0 : (x > cap ? cap : x)) : 0u;
    }
    for (uint32_t b = tid; b < B; b += 256) {
      const int64_t L = (int64_t)(S[b + 1] - S[b]);
      const int64_t x = lo - (int64_t)S[b];
      co[b] = used ? (uint32_t)(x < 0 ? 0 : (x > L ? L : x)) : 0u;
    }
    if (tid == 0) {
      const int64_t x = total - lo;
      a.buffer_lengths[r] = used ? (int32_t)(x > cap ? cap : x) : -1;
    }
  }
}

// Gather of wide rows (>= 32 copy units): each wave copies whole buffer slots,
// GATHER_ROWS of them per step.  A slot's
// sequence (binary search of the row's slice starts), cache position and
// physical page are found once per slot in scalar registers; the 64 lanes then
// walk the slot in UNIT-byte pieces, with all of the step's loads in flight
// before its stores.
template <typename T>
__device__ __forceinline__ T ld_unit(const uint8_t* p) { return *reinterpret_cast<const T*>(p); }
template <typename T>
__device__ __forceinline__ void st_unit(uint8_t* p, T v) {
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));   // streamed: the buffer is not re-read here
}
template <int UNIT> struct UnitType;
template <> struct UnitType<16> { typedef i32x4 T; };
template <> struct UnitType<8> { typedef uint64_t T; };
template <> struct UnitType<4> { typedef uint32_t T; };
template <> struct UnitType<2> { typedef uint16_t T; };
template <> struct UnitType<1> { typedef uint8_t T; };

constexpr int GATHER_ROWS = 8;

template <int UNIT>
__global__ void __launch_bounds__(256) gather_rows_kernel(GatherArgs a) {
  typedef typename UnitType<UNIT>::T T;
  extern __shared__ uint32_t bro[];           // [B + 1] slice starts of this row
  const uint32_t B = a.batch;
  for (uint32_t b = threadIdx.x; b <= B; b += 256) bro[b] = a.buffer_row_offsets[b];
  __syncthreads();
  // page table and cache offsets through the constant address space: the
  // per-slot lookups are uniform, so they become scalar loads
  typedef const __attribute__((address_space(4))) uint32_t CU32;
  CU32* const PT = (CU32*)a.page_table;
  CU32* const CO = (CU32*)a.cache_offsets;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = blockIdx.x * 4u + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nwaves = gridDim.x * 4u;
  const uint32_t first = __builtin_amdgcn_readfirstlane(bro[0]);
  const uint32_t total = __builtin_amdgcn_readfirstlane(bro[B]);
  const uint32_t upr = (uint32_t)(a.copy_bytes / UNIT);
  for (uint32_t s0 = first + wave * GATHER_ROWS; s0 < total; s0 += nwaves * GATHER_ROWS) {
    const uint8_t* src[GATHER_ROWS];
    uint8_t* dst[GATHER_ROWS];
    bool ok[GATHER_ROWS];
    // sequence of the step's first slot: last b with bro[b] <= slot (binary search),
    // then walk forward for the following slots
    uint32_t lo = 0, hi = B;                  // invariant: bro[lo] <= s0 < bro[hi]
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(bro[mid]) <= s0) lo = mid; else hi = mid;
    }
    uint32_t next_start = __builtin_amdgcn_readfirstlane(bro[lo + 1]);
#pragma unroll
    for (int r = 0; r < GATHER_ROWS; ++r) {
      const uint32_t slot = s0 + r;
      ok[r] = slot < total;
      while (ok[r] && slot >= next_start) {
        ++lo;
        next_start = __builtin_amdgcn_readfirstlane(bro[lo + 1]);
      }
      // a slot past the row's last one has no position: its page is not looked up
      // (its position could lie past the last sequence's page-table row)
      const uint32_t pos = ok[r] ? CO[lo] + (slot - __builtin_amdgcn_readfirstlane(bro[lo])) : 0u;
      const uint32_t page = ok[r] ? PT[(size_t)lo * a.max_pages + pos / a.page_size] : 0u;
      const size_t row = (size_t)page * a.page_size + pos % a.page_size;
      src[r] = a.cache + row * a.row_bytes + a.col_bytes;
      dst[r] = a.out + (size_t)slot * a.copy_bytes;
    }
    for (uint32_t c = lane; c < upr; c += 64u) {
      T v[GATHER_ROWS];
#pragma unroll
      for (int r = 0; r < GATHER_ROWS; ++r)
        if (ok[r]) v[r] = ld_unit<T>(src[r] + (size_t)c * UNIT);
#pragma unroll
      for (int r = 0; r < GATHER_ROWS; ++r)
        if (ok[r]) st_unit<T>(dst[r] + (size_t)c * UNIT, v[r]);
    }
  }
}

// Gather of narrow rows: one thread per copy unit (UNIT bytes) of a buffer slot; consecutive threads
// walk along a row so both the page read and the buffer write are coalesced.
template <int UNIT>
__global__ void __launch_bounds__(256) gather_kernel(GatherArgs a) {
  extern __shared__ uint32_t bro[];           // [B + 1] slice starts of this row
  const uint32_t B = a.batch;
  for (uint32_t b = threadIdx.x; b <= B; b += 256) bro[b] = a.buffer_row_offsets[b];
  __syncthreads();
  const uint64_t units_per_row = a.copy_bytes / UNIT;
  const uint64_t total_units = (uint64_t)bro[B] * units_per_row;
  for (uint64_t u = (uint64_t)blockIdx.x * 256 + threadIdx.x; u < total_units; u += (uint64_t)gridDim.x * 256) {
    const uint32_t slot = (uint32_t)(u / units_per_row);
    const uint32_t c = (uint32_t)(u - (uint64_t)slot * units_per_row);
    if (slot < bro[0]) continue;              // not part of any sequence's slice
    // sequence owning the slot: last b with bro[b] <= slot (empty slices skipped)
    uint32_t lo = 0, hi = B;                  // invariant: bro[lo] <= slot < bro[hi]
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (bro[mid] <= slot) lo = mid; else hi = mid;
    }
    const uint32_t b = lo;
    const uint32_t pos = a.cache_offsets[b] + (slot - bro[b]);
    const uint32_t page = a.page_table[(size_t)b * a.max_pages + pos / a.page_size];
    const size_t row = (size_t)page * a.page_size + pos % a.page_size;
    const uint8_t* src = a.cache + row * a.row_bytes + a.col_bytes + (size_t)c * UNIT;
    uint8_t* dst = a.out + (size_t)slot * a.copy_bytes + (size_t)c * UNIT;
    if constexpr (UNIT == 16) st16(dst, ld16(src));
    else if constexpr (UNIT == 8) *reinterpret_cast<uint64_t*>(dst) = *reinterpret_cast<const uint64_t*>(src);
    else if constexpr (UNIT == 4) *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
    else if constexpr (UNIT == 2) *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(src);
    else *dst = *src;
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  const uint32_t rows_per_block = 16;
  const uint32_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  PlanArgs args = a;
  args.rows_per_block = rows_per_block;
  const size_t lds = sizeof(uint64_t) * (a.batch + 1);
  hipLaunchKernelGGL(plan_kernel, dim3(blocks), dim3(256), lds, stream, args);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, int unit, hipStream_t stream) {
  const size_t lds = sizeof(uint32_t) * (a.batch + 1);
  if (a.copy_bytes / unit >= 32) {                     // wide rows: a wave per slot
    const uint64_t waves = ((uint64_t)a.cap + GATHER_ROWS - 1) / GATHER_ROWS;
    uint64_t blocks = (waves + 3) / 4;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    switch (unit) {
      case 16: hipLaunchKernelGGL(gather_rows_kernel<16>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
      case 8: hipLaunchKernelGGL(gather_rows_kernel<8>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
      case 4: hipLaunchKernelGGL(gather_rows_kernel<4>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
      case 2: hipLaunchKernelGGL(gather_rows_kernel<2>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
      default: hipLaunchKernelGGL(gather_rows_kernel<1>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
    }
    return hipGetLastError();
  }
  const uint64_t units = (uint64_t)a.cap * (a.copy_bytes / unit);
  uint64_t blocks = (units + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks == 0) blocks = 1;
  switch (unit) {
    case 16: hipLaunchKernelGGL(gather_kernel<16>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
    case 8: hipLaunchKernelGGL(gather_kernel<8>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
    case 4: hipLaunchKernelGGL(gather_kernel<4>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
    case 2: hipLaunchKernelGGL(gather_kernel<2>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
    default: hipLaunchKernelGGL(gather_kernel<1>, dim3((uint32_t)blocks), dim3(256), lds, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace mla
