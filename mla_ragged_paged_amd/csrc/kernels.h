// Kernel argument blocks and launchers of the MLA prefill library (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct PlanArgs {
  const uint32_t* input_row_offsets;  // [B+1]
  const uint32_t* cache_lengths;      // [B]
  uint32_t batch;
  uint32_t cap;
  uint32_t rows;
  uint32_t rows_per_block;
  uint32_t* buffer_row_offsets;       // [rows][B+1]
  uint32_t* cache_offsets;            // [rows][B]
  int32_t* buffer_lengths;            // [rows]
  int32_t* status;                    // nullable
};

struct GatherArgs {
  const uint8_t* cache;               // layer base, [pages][page_size][1][row_width] elements
  const uint32_t* page_table;         // [B][max_pages]
  const uint32_t* buffer_row_offsets; // [B+1]
  const uint32_t* cache_offsets;      // [B]
  uint8_t* out;                       // [cap][copy_bytes]
  uint64_t row_bytes;                 // bytes of one cache row
  uint64_t col_bytes;                 // byte offset of the copied window in a row
  uint64_t copy_bytes;                // bytes copied per row
  uint32_t max_pages;
  uint32_t page_size;
  uint32_t batch;
  uint32_t cap;
};

struct PrefillArgs {
  void* out;                          // [T][H][128], bf16 or fp32 (out_fp32)
  float* lse;                         // [T][H] log-sum-exp (natural log) or nullptr
  const float* prev_out;              // [T][H][128] fp32 earlier partial or nullptr
  const float* prev_lse;              // [T][H] its log-sum-exp (with prev_out)
  const void* q;                      // [T][H][192]
  const void* k_nope;                 // [rows][H][128]
  const void* v;                      // [rows][H][128]
  const void* cache;                  // layer base, [pages][page_size][1][row_width]
  const uint32_t* page_table;         // [B][max_pages]
  const uint32_t* cache_lengths;      // [B]
  const uint32_t* valid_length;       // [B+1]
  const uint32_t* cache_row_offsets;  // [B+1]
  const uint32_t* cache_offsets;      // [B] or nullptr
  const float* q_scale;               // fp8 only
  const float* k_nope_scale;
  const float* v_scale;
  const float* k_rope_scale;
  uint32_t max_pages;
  uint32_t page_size;
  uint32_t page_shift;                // log2(page_size) when a power of two, else 0xFFFFFFFF
  uint32_t row_width;                 // elements per cache row
  uint32_t rope_col;
  uint32_t cache_bytes;               // bytes of one layer of the cache (< 4 GiB)
  uint32_t batch;
  uint32_t heads;
  uint32_t qtiles;                    // query tiles per sequence (launch bound)
  uint32_t out_fp32;                  // 1: out is fp32, 0: bf16
  uint32_t causal;                    // 1: key visible iff kpos <= qpos; 0: every key visible
  float scale;                        // softmax scale (its sign is applied to Q)
  float scale_log2;                   // max(|scale| * log2(e), 1e-30)
  float* acc;                         // row mode: [T][H][128] fp32 partial carried between rows
  float* acc_lse;                     // row mode: [T][H]
  uint32_t row_mode;                  // 1: one plan row of several, called in row order
  const void* q_rope;                 // split Q: bf16 [T][H][64] (q then holds q_nope [T][H][128])
  const void* rope_rows;              // contiguous K_rope [rows][64] laid out like K (bf16, or e4m3 with
                                      // k_rope_scale), or nullptr (paged)
  uint32_t q_split;                   // 1: Q comes as q_nope (a.q) + q_rope
  float* ws;                          // key split: [2][T][H][128] fp32 partial rows, then [2][T][H] lse
  uint32_t split_keys;                // key split: tiles seeing more keys are split in two; 0 = none
  uint32_t tokens;                    // T (key split: workspace plane size)
};

struct MergeArgs {
  void* out;                          // [rows][128], bf16 or fp32 (out_fp32)
  float* lse;                         // [rows] or nullptr
  const float* o_a;                   // [rows][128]
  const float* lse_a;                 // [rows]
  const float* o_b;
  const float* lse_b;
  uint64_t rows;                      // tokens * heads
  uint32_t out_fp32;
};

struct LatentArgs {
  const uint8_t* cache;               // layer base, [pages][page_size][1][row_width] bf16
  const uint32_t* page_table;         // [B][max_pages]
  const uint32_t* bro;                // [B+1] one plan row's buffer_row_offsets
  const uint32_t* co;                 // [B]   its cache_offsets
  const uint16_t* w;                  // [H*256][latent_dim] bf16
  uint16_t* k_nope;                   // [cap][H][128] bf16
  uint16_t* v;                        // [cap][H][128] bf16
  uint32_t max_pages;
  uint32_t page_size;
  uint32_t page_shift;                // log2(page_size) when a power of two, else 0xFFFFFFFF
  uint32_t row_bytes;                 // bytes of one cache row
  uint32_t latent_col;                // first latent column of a cache row
  uint32_t latent_dim;                // latent columns (a multiple of 64)
  uint32_t cache_bytes;               // bytes of one layer (< 4 GiB)
  uint32_t batch;
  uint32_t heads;
  uint32_t cap;                       // slots of K_nope / V
};

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, int unit, hipStream_t stream);
hipError_t launch_prefill_bf16(PrefillArgs a, uint32_t q_max, hipStream_t stream);
hipError_t launch_prefill_fp8(PrefillArgs a, uint32_t q_max, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_kv_split_merge(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_latent_up(const LatentArgs& a, hipStream_t stream);

}  // namespace mla
