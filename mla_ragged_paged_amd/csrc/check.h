// Argument block and launcher of the device-side precondition check (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Violation bits of the device-side precondition check (the public
// MLA_VIOLATION_* values).
constexpr uint32_t CHECK_Q_OFFSETS = 1;
constexpr uint32_t CHECK_ROW_OFFSETS = 2;
constexpr uint32_t CHECK_POSITIONS = 4;
constexpr uint32_t CHECK_PAGE_IDS = 8;

struct CheckArgs {
  const uint32_t* valid_length;       // [B+1] new-token offsets, or nullptr
  const uint32_t* cache_lengths;      // [B] p_b (read with valid_length)
  const uint32_t* page_table;         // [B][max_pages], or nullptr (no paged reads)
  const uint32_t* row_offsets;        // [B+1] one buffer row's offsets, or nullptr
  const uint32_t* row_positions;      // [B] its first cache positions, or nullptr (0)
  int32_t* violations;                // ORed with the violated bits
  uint32_t batch;
  uint32_t tokens;                    // T, checked against valid_length[B] when tokens_known
  uint32_t tokens_known;
  uint32_t q_max;                     // 0: unchecked
  uint32_t row_capacity;              // 0: unchecked
  uint32_t max_pages;
  uint32_t page_size;
  uint32_t num_pages;
};

hipError_t launch_check(const CheckArgs& a, hipStream_t stream);

}  // namespace mla
