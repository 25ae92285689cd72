// C ABI of the MLA prefill library: host-side validation, launch geometry and
// dtype dispatch.  Declarations and the full contract live in mla_prefill.h.
#include "mla_prefill.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "check.h"
#include "kernels.h"

static_assert(mla::CHECK_Q_OFFSETS == MLA_VIOLATION_Q_OFFSETS && mla::CHECK_ROW_OFFSETS == MLA_VIOLATION_ROW_OFFSETS &&
                  mla::CHECK_POSITIONS == MLA_VIOLATION_POSITIONS && mla::CHECK_PAGE_IDS == MLA_VIOLATION_PAGE_IDS,
              "violation bits");

namespace {

thread_local int g_last_hip_error = 0;

// ---- debug mode: every call checks its device data first (mla_prefill_set_debug)
int debug_from_env() {
  const char* e = std::getenv("MLA_PREFILL_DEBUG");
  return e && std::strcmp(e, "1") == 0 ? 1 : 0;
}
std::atomic<int> g_debug{debug_from_env()};
std::mutex g_debug_mu;                 // one check at a time: the flag of a GPU is shared
constexpr int MAX_DEVICES = 64;
int32_t* g_debug_flag[MAX_DEVICES] = {};

// Launch-failure injection for tests of the error path: when the environment
// variable MLA_PREFILL_FAIL_LAUNCH holds a nonzero HIP error code as the library
// loads, every call that passes its host-side checks returns MLA_ERR_HIP with
// that code instead of enqueueing anything.
int fail_launch_from_env() {
  const char* e = std::getenv("MLA_PREFILL_FAIL_LAUNCH");
  return e ? std::atoi(e) : 0;
}
const int g_fail_launch = fail_launch_from_env();

mla_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  g_last_hip_error = (int)e;
  return MLA_ERR_HIP;
}

size_t dtype_bytes(mla_dtype_t t) { return t == MLA_FP8_E4M3FN ? 1 : t == MLA_FP32 ? 4 : 2; }

bool dtype_known(mla_dtype_t t) { return t == MLA_BF16 || t == MLA_FP8_E4M3FN; }

mla_status_t check_cache(const mla_paged_cache_t* kv, uint32_t layer_idx) {
  if (!kv) return MLA_ERR_NULL_ARG;
  if (!kv->data || !kv->page_table || !kv->cache_lengths) return MLA_ERR_NULL_ARG;
  if (!dtype_known(kv->dtype)) return MLA_ERR_UNSUPPORTED_DTYPE;
  if (kv->num_layers == 0 || layer_idx >= kv->num_layers || kv->num_pages == 0 || kv->page_size == 0 ||
      kv->row_width == 0 || kv->max_pages_per_seq == 0)
    return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}

// Runs the device-side check of a call's arguments when debug mode is on: the
// check kernel on the call's stream, then a wait for its flag.  No launch and
// no wait when debug mode is off.
mla_status_t debug_check(mla::CheckArgs c, void* stream) {
  if (g_fail_launch != 0) return hip_status(static_cast<hipError_t>(g_fail_launch));
  if (g_debug.load(std::memory_order_relaxed) == 0 || c.batch == 0) return MLA_OK;
  std::lock_guard<std::mutex> lock(g_debug_mu);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the flag lives on the stream's GPU (the current one for the null stream)
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= MAX_DEVICES) return MLA_ERR_BAD_SHAPE;
  if (!g_debug_flag[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&g_debug_flag[dev]), sizeof(int32_t));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return hip_status(e);
  }
  static const int32_t zero = 0;
  int32_t found = 0;
  c.violations = g_debug_flag[dev];
  e = hipMemcpyAsync(c.violations, &zero, sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = mla::launch_check(c, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&found, c.violations, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e);
  return found ? MLA_ERR_PRECONDITION : MLA_OK;
}

// Check arguments with the paged-cache fields of a descriptor (page table
// optional) and nothing else set.
mla::CheckArgs check_args(const mla_paged_cache_t* kv, uint32_t batch) {
  mla::CheckArgs c{};
  c.batch = batch;
  c.cache_lengths = kv->cache_lengths;
  if (kv->page_table && kv->page_size && kv->max_pages_per_seq && kv->num_pages) {
    c.page_table = kv->page_table;
    c.max_pages = kv->max_pages_per_seq;
    c.page_size = kv->page_size;
    c.num_pages = kv->num_pages;
  }
  return c;
}

// ---- scratch of mla_prefill_ragged_kvsplit_noalloc: the key split's fp32
// partial rows and log-sum-exps, in a device array of this library (each GPU
// the library runs on holds its own copy until the process ends).  Host code
// uses the array only through the device address hipGetSymbolAddress gives for
// each GPU, looked up on the first call on that GPU.
static __device__ __align__(256) float scratch[MLA_NOALLOC_SCRATCH_BYTES / sizeof(float)];
std::mutex g_scratch_mu;
float* g_scratch_ptr[MAX_DEVICES] = {};

hipError_t scratch_of_stream(hipStream_t s, float** out) {
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

const uint8_t* layer_base(const mla_paged_cache_t* kv, uint32_t layer_idx) {
  return static_cast<const uint8_t*>(kv->data) +
         (size_t)layer_idx * kv->num_pages * kv->page_size * kv->row_width * dtype_bytes(kv->dtype);
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL_ARG: return "MLA_ERR_NULL_ARG: a required pointer is NULL";
    case MLA_ERR_BAD_SHAPE: return "MLA_ERR_BAD_SHAPE: inconsistent or unsupported sizes";
    case MLA_ERR_UNSUPPORTED_DTYPE: return "MLA_ERR_UNSUPPORTED_DTYPE: dtype combination not offered";
    case MLA_ERR_UNSUPPORTED_DIMS: return "MLA_ERR_UNSUPPORTED_DIMS: q_depth must be 192 and depth 128";
    case MLA_ERR_UNSUPPORTED_MASK: return "MLA_ERR_UNSUPPORTED_MASK: the mask is neither causal nor null";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: the HIP runtime reported an error";
    case MLA_ERR_PRECONDITION:
      return "MLA_ERR_PRECONDITION: the device data violate a documented precondition (debug mode)";
  }
  return "unknown mla_status_t";
}

int mla_prefill_last_hip_error(void) { return g_last_hip_error; }

int mla_prefill_set_debug(int on) { return g_debug.exchange(on ? 1 : 0); }

mla_status_t mla_prefill_check(const mla_paged_cache_t* kv, const uint32_t* valid_length, uint32_t batch_size,
                               uint32_t total_q_tokens, uint32_t q_max_seq_len, const uint32_t* row_offsets,
                               const uint32_t* row_positions, uint32_t row_capacity, int32_t* violations,
                               void* stream) {
  if (!kv || !kv->cache_lengths || !violations) return MLA_ERR_NULL_ARG;
  if (!valid_length && !row_offsets) return MLA_ERR_NULL_ARG;
  if (batch_size > MLA_MAX_BATCH) return MLA_ERR_BAD_SHAPE;
  if (kv->page_table && (kv->page_size == 0 || kv->max_pages_per_seq == 0 || kv->num_pages == 0))
    return MLA_ERR_BAD_SHAPE;
  if (batch_size == 0) return MLA_OK;
  mla::CheckArgs c = check_args(kv, batch_size);
  c.valid_length = valid_length;
  c.tokens = total_q_tokens;
  c.tokens_known = total_q_tokens != 0xFFFFFFFFu ? 1u : 0u;
  c.q_max = q_max_seq_len;
  c.row_offsets = row_offsets;
  c.row_positions = row_positions;
  c.row_capacity = row_capacity;
  c.violations = violations;
  if (g_fail_launch != 0) return hip_status(static_cast<hipError_t>(g_fail_launch));
  return hip_status(mla::launch_check(c, static_cast<hipStream_t>(stream)));
}

mla_status_t mla_prefill_plan(const uint32_t* input_row_offsets, uint32_t batch_size, const mla_paged_cache_t* kv,
                              uint32_t layer_idx, uint32_t buffer_token_size, uint32_t num_buffer_rows,
                              uint32_t* buffer_row_offsets, uint32_t* cache_offsets, int32_t* buffer_lengths,
                              int32_t* device_status, void* stream) {
  if (!input_row_offsets || !kv || !buffer_row_offsets || !cache_offsets || !buffer_lengths) return MLA_ERR_NULL_ARG;
  if (!kv->cache_lengths) return MLA_ERR_NULL_ARG;
  if (kv->num_layers == 0 || layer_idx >= kv->num_layers) return MLA_ERR_BAD_SHAPE;
  if (buffer_token_size == 0 || buffer_token_size > 0x7FFFFFFFu || num_buffer_rows == 0) return MLA_ERR_BAD_SHAPE;
  if (batch_size > MLA_MAX_BATCH) return MLA_ERR_BAD_SHAPE;
  {
    // the whole batch: offsets, and the pages of every position a later gather reads
    mla::CheckArgs c = check_args(kv, batch_size);
    c.valid_length = input_row_offsets;
    mla_status_t st = debug_check(c, stream);
    if (st != MLA_OK) return st;
  }
  mla::PlanArgs a{};
  a.input_row_offsets = input_row_offsets;
  a.cache_lengths = kv->cache_lengths;
  a.batch = batch_size;
  a.cap = buffer_token_size;
  a.rows = num_buffer_rows;
  a.buffer_row_offsets = buffer_row_offsets;
  a.cache_offsets = cache_offsets;
  a.buffer_lengths = buffer_lengths;
  a.status = device_status;
  if (g_fail_launch != 0) return hip_status(static_cast<hipError_t>(g_fail_launch));
  return hip_status(mla::launch_plan(a, static_cast<hipStream_t>(stream)));
}

mla_status_t mla_prefill_gather(const mla_paged_cache_t* kv, uint32_t layer_idx, uint32_t batch_size,
                                const uint32_t* buffer_row_offsets_r, const uint32_t* cache_offsets_r,
                                uint32_t col_begin, uint32_t col_count, uint32_t buffer_token_size, void* out,
                                void* stream) {
  mla_status_t st = check_cache(kv, layer_idx);
  if (st != MLA_OK) return st;
  if (!buffer_row_offsets_r || !cache_offsets_r || !out) return MLA_ERR_NULL_ARG;
  if (batch_size == 0) return MLA_OK;
  if (batch_size > MLA_MAX_BATCH || col_count == 0 || (uint64_t)col_begin + col_count > kv->row_width ||
      buffer_token_size == 0)
    return MLA_ERR_BAD_SHAPE;
  {
    mla::CheckArgs c = check_args(kv, batch_size);
    c.row_offsets = buffer_row_offsets_r;
    c.row_positions = cache_offsets_r;
    c.row_capacity = buffer_token_size;
    st = debug_check(c, stream);
    if (st != MLA_OK) return st;
  }
  const size_t el = dtype_bytes(kv->dtype);
  mla::GatherArgs a{};
  a.cache = layer_base(kv, layer_idx);
  a.page_table = kv->page_table;
  a.buffer_row_offsets = buffer_row_offsets_r;
  a.cache_offsets = cache_offsets_r;
  a.out = static_cast<uint8_t*>(out);
  a.row_bytes = (uint64_t)kv->row_width * el;
  a.col_bytes = (uint64_t)col_begin * el;
  a.copy_bytes = (uint64_t)col_count * el;
  a.max_pages = kv->max_pages_per_seq;
  a.page_size = kv->page_size;
  a.batch = batch_size;
  a.cap = buffer_token_size;
  // widest copy unit that every address and size is a multiple of
  int unit = 16;
  while (unit > 1 && ((a.row_bytes % unit) || (a.col_bytes % unit) || (a.copy_bytes % unit) ||
                      (reinterpret_cast<uintptr_t>(a.cache) % unit) || (reinterpret_cast<uintptr_t>(out) % unit)))
    unit >>= 1;
  if (g_fail_launch != 0) return hip_status(static_cast<hipError_t>(g_fail_launch));
  return hip_status(mla::launch_gather(a, unit, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Query and K_rope sources of a call: one q [T][H][192], or (split) q_nope
// [T][H][128] + bf16 q_rope [T][H][64]; K_rope from the paged cache, or from
// contiguous rows laid out like K (their element type and scale in the cache
// descriptor's dtype and scale).
struct QuerySource {
  const void* q;           // q, or q_nope when split
  const void* q_rope;      // split only
  const void* rope_rows;   // NULL: K_rope from the paged cache
  bool split;
};

// Key split of a call: tiles seeing more than split_keys keys are computed in two
// halves into the workspace and merged (split_keys 0: none).
struct KvSplit {
  uint32_t split_keys;
  float* workspace;
  uint64_t workspace_bytes;
};

// Shared validation and launch of the attention entry points.
mla_status_t prefill_impl(void* output, mla_dtype_t output_dtype, float* lse, const float* prev_output,
                          const float* prev_lse, float* acc, float* acc_lse, bool row_mode, const QuerySource& qs,
                          mla_dtype_t qkv_dtype, const void* k_nope, const void* v, const mla_paged_cache_t* k_rope,
                          uint32_t layer_idx, const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                          const uint32_t* cache_offsets, uint32_t batch_size, uint32_t total_q_tokens,
                          uint32_t num_heads, uint32_t q_depth, uint32_t depth, mla_mask_t mask, float scale,
                          const float* q_scale, const float* k_nope_scale, const float* v_scale,
                          uint32_t q_max_seq_len, void* stream, const KvSplit& kvs = KvSplit{0u, nullptr, 0u},
                          bool debug_allowed = true) {
  if (!output || !qs.q || !k_nope || !v || !valid_length || !cache_row_offsets) return MLA_ERR_NULL_ARG;
  if (kvs.split_keys != 0) {
    if (!kvs.workspace) return MLA_ERR_NULL_ARG;
    if (kvs.split_keys < 128 || reinterpret_cast<uintptr_t>(kvs.workspace) % 16 ||
        kvs.workspace_bytes < mla_prefill_kvsplit_workspace_bytes(total_q_tokens, num_heads))
      return MLA_ERR_BAD_SHAPE;
  }
  if (qs.split && !qs.q_rope) return MLA_ERR_NULL_ARG;
  if ((prev_output == nullptr) != (prev_lse == nullptr)) return MLA_ERR_NULL_ARG;
  if (row_mode && (!acc || !acc_lse)) return MLA_ERR_NULL_ARG;
  const bool contig = qs.rope_rows != nullptr;
  if (contig) {
    // K_rope rows are given; the cache descriptor supplies the start positions
    // and the rows' element type and scale
    if (!k_rope || !k_rope->cache_lengths) return MLA_ERR_NULL_ARG;
    if (!dtype_known(k_rope->dtype)) return MLA_ERR_UNSUPPORTED_DTYPE;
  } else {
    mla_status_t st = check_cache(k_rope, layer_idx);
    if (st != MLA_OK) return st;
  }
  if (q_depth != (qs.split ? 128u : 192u) || depth != 128) return MLA_ERR_UNSUPPORTED_DIMS;
  if (mask != MLA_MASK_CAUSAL && mask != MLA_MASK_NULL) return MLA_ERR_UNSUPPORTED_MASK;
  if (!dtype_known(qkv_dtype) || (output_dtype != MLA_BF16 && output_dtype != MLA_FP32))
    return MLA_ERR_UNSUPPORTED_DTYPE;
  const bool fp8 = qkv_dtype == MLA_FP8_E4M3FN;
  // K_rope's type: the descriptor's (it must match q's for a full query; a split
  // query takes bf16 K_rope, or e4m3 K_rope with e4m3 q_nope)
  const bool rope_fp8 = k_rope->dtype == MLA_FP8_E4M3FN;
  if (!qs.split && k_rope->dtype != qkv_dtype) return MLA_ERR_UNSUPPORTED_DTYPE;
  if (qs.split && rope_fp8 && !fp8) return MLA_ERR_UNSUPPORTED_DTYPE;
  if (fp8 && (!q_scale || !k_nope_scale || !v_scale)) return MLA_ERR_NULL_ARG;
  if (rope_fp8 && !k_rope->scale) return MLA_ERR_NULL_ARG;
  if (!fp8 && (q_scale || k_nope_scale || v_scale)) return MLA_ERR_UNSUPPORTED_DTYPE;
  if (batch_size == 0 || total_q_tokens == 0) return MLA_OK;
  if (num_heads == 0) return MLA_ERR_BAD_SHAPE;
  const uint32_t el = (uint32_t)dtype_bytes(qkv_dtype);
  uint64_t layer_bytes = 0;
  if (!contig) {
    // 16-byte row segments: the rope window and rows must start on 16-byte boundaries
    const uint32_t rel = (uint32_t)dtype_bytes(k_rope->dtype);
    if ((k_rope->rope_col * rel) % 16 || (k_rope->row_width * rel) % 16 ||
        (uint64_t)k_rope->rope_col + 64 > k_rope->row_width)
      return MLA_ERR_BAD_SHAPE;
    layer_bytes = (uint64_t)k_rope->num_pages * k_rope->page_size * k_rope->row_width * rel;
    if (reinterpret_cast<uintptr_t>(k_rope->data) % 16) return MLA_ERR_BAD_SHAPE;
  }
  if ((reinterpret_cast<uintptr_t>(qs.q) | reinterpret_cast<uintptr_t>(qs.q_rope) |
       reinterpret_cast<uintptr_t>(qs.rope_rows) | reinterpret_cast<uintptr_t>(k_nope) |
       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(output) |
       reinterpret_cast<uintptr_t>(prev_output) | reinterpret_cast<uintptr_t>(acc)) % 16 ||
      (reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(prev_lse) |
       reinterpret_cast<uintptr_t>(acc_lse)) % 4)
    return MLA_ERR_BAD_SHAPE;
  // the kernels address one sequence's rows and one cache layer with 32-bit byte offsets
  if (layer_bytes >= (1ull << 32) || (uint64_t)total_q_tokens * num_heads * q_depth * el >= (1ull << 32) ||
      (qs.split && (uint64_t)total_q_tokens * num_heads * 64 * 2 >= (1ull << 32)))
    return MLA_ERR_BAD_SHAPE;
  const uint32_t q_max = q_max_seq_len ? q_max_seq_len : total_q_tokens;
  // launch units (two per query tile with the key split), counted in 32 bits on the device
  const uint64_t units = (uint64_t)num_heads * batch_size * ((q_max + 127) / 128) * (kvs.split_keys ? 2u : 1u);
  if (units > 0x7FFFFFF0ull) return MLA_ERR_BAD_SHAPE;

  {
    // this row's keys (and, through the page table, their K_rope rows)
    mla::CheckArgs c = check_args(k_rope, batch_size);
    if (contig) c.page_table = nullptr;
    c.valid_length = valid_length;
    c.tokens = total_q_tokens;
    c.tokens_known = 1u;
    c.q_max = q_max_seq_len;
    c.row_offsets = cache_row_offsets;
    c.row_positions = cache_offsets;
    mla_status_t st = debug_allowed ? debug_check(c, stream) : MLA_OK;
    if (st != MLA_OK) return st;
  }
  mla::PrefillArgs a{};
  a.out = output;
  a.lse = lse;
  a.prev_out = prev_output;
  a.prev_lse = prev_lse;
  a.acc = acc;
  a.acc_lse = acc_lse;
  a.row_mode = row_mode ? 1u : 0u;
  a.out_fp32 = output_dtype == MLA_FP32 ? 1u : 0u;
  a.causal = mask == MLA_MASK_CAUSAL ? 1u : 0u;
  a.q = qs.q;
  a.q_rope = qs.q_rope;
  a.rope_rows = qs.rope_rows;
  // 0: full query; 1: split, e4m3 K_rope from the cache; 2: split, bf16 K_rope
  a.q_split = !qs.split ? 0u : rope_fp8 ? 1u : 2u;
  a.k_nope = k_nope;
  a.v = v;
  a.cache_lengths = k_rope->cache_lengths;
  a.k_rope_scale = k_rope->scale;
  if (!contig) {
    a.cache = layer_base(k_rope, layer_idx);
    a.page_table = k_rope->page_table;
    a.max_pages = k_rope->max_pages_per_seq;
    a.page_size = k_rope->page_size;
    a.page_shift = (k_rope->page_size & (k_rope->page_size - 1)) == 0 ? (uint32_t)__builtin_ctz(k_rope->page_size)
                                                                        : 0xFFFFFFFFu;
    a.row_width = k_rope->row_width;
    a.rope_col = k_rope->rope_col;
    a.cache_bytes = (uint32_t)layer_bytes;
  }
  a.valid_length = valid_length;
  a.cache_row_offsets = cache_row_offsets;
  a.cache_offsets = cache_offsets;
  a.q_scale = q_scale;
  a.k_nope_scale = k_nope_scale;
  a.v_scale = v_scale;
  a.batch = batch_size;
  a.heads = num_heads;
  a.tokens = total_q_tokens;
  a.split_keys = kvs.split_keys;
  a.ws = kvs.workspace;
  a.scale = scale;
  {
    const float c = (scale < 0.f ? -scale : scale) * 1.4426950408889634f;
    a.scale_log2 = c > 1e-30f ? c : 1e-30f;  // scale 0: every visible key weighs the same
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g_fail_launch != 0) return hip_status(static_cast<hipError_t>(g_fail_launch));
  if (fp8) return hip_status(mla::launch_prefill_fp8(a, q_max, s));
  return hip_status(mla::launch_prefill_bf16(a, q_max, s));
}

}  // namespace

extern "C" {

mla_status_t mla_prefill_ragged_lse(void* output, mla_dtype_t output_dtype, float* lse, const float* prev_output,
                                    const float* prev_lse, const void* q, mla_dtype_t qkv_dtype, const void* k_nope,
                                    const void* v, const mla_paged_cache_t* k_rope, uint32_t layer_idx,
                                    const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                    const uint32_t* cache_offsets, uint32_t batch_size, uint32_t total_q_tokens,
                                    uint32_t num_heads, uint32_t q_depth, uint32_t depth, mla_mask_t mask,
                                    float scale, const float* q_scale, const float* k_nope_scale,
                                    const float* v_scale, uint32_t q_max_seq_len, void* stream) {
  return prefill_impl(output, output_dtype, lse, prev_output, prev_lse, nullptr, nullptr, false,
                      QuerySource{q, nullptr, nullptr, false}, qkv_dtype, k_nope,
                      v, k_rope, layer_idx, valid_length, cache_row_offsets, cache_offsets, batch_size,
                      total_q_tokens, num_heads, q_depth, depth, mask, scale, q_scale, k_nope_scale, v_scale,
                      q_max_seq_len, stream);
}

mla_status_t mla_prefill_ragged_row(void* output, mla_dtype_t output_dtype, float* lse, float* acc, float* acc_lse,
                                    const void* q, mla_dtype_t qkv_dtype, const void* k_nope, const void* v,
                                    const mla_paged_cache_t* k_rope, uint32_t layer_idx,
                                    const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                    const uint32_t* cache_offsets, uint32_t batch_size, uint32_t total_q_tokens,
                                    uint32_t num_heads, uint32_t q_depth, uint32_t depth, mla_mask_t mask,
                                    float scale, const float* q_scale, const float* k_nope_scale,
                                    const float* v_scale, uint32_t q_max_seq_len, void* stream) {
  return prefill_impl(output, output_dtype, lse, nullptr, nullptr, acc, acc_lse, true,
                      QuerySource{q, nullptr, nullptr, false}, qkv_dtype, k_nope, v,
                      k_rope, layer_idx, valid_length, cache_row_offsets, cache_offsets, batch_size, total_q_tokens,
                      num_heads, q_depth, depth, mask, scale, q_scale, k_nope_scale, v_scale, q_max_seq_len, stream);
}

mla_status_t mla_prefill_ragged_row_krope(void* output, mla_dtype_t output_dtype, float* lse, float* acc,
                                          float* acc_lse, const void* q, mla_dtype_t qkv_dtype, const void* k_nope,
                                          const void* v, const void* k_rope, const float* k_rope_scale,
                                          const uint32_t* cache_lengths, const uint32_t* valid_length,
                                          const uint32_t* cache_row_offsets, const uint32_t* cache_offsets,
                                          uint32_t batch_size, uint32_t total_q_tokens, uint32_t num_heads,
                                          uint32_t q_depth, uint32_t depth, mla_mask_t mask, float scale,
                                          const float* q_scale, const float* k_nope_scale, const float* v_scale,
                                          uint32_t q_max_seq_len, void* stream) {
  if (!k_rope || !cache_lengths) return MLA_ERR_NULL_ARG;
  // the rows' element type is the query's; the descriptor carries only the start
  // positions and the rows' scale
  mla_paged_cache_t rows{};
  rows.dtype = qkv_dtype;
  rows.cache_lengths = cache_lengths;
  rows.scale = k_rope_scale;
  if (qkv_dtype != MLA_FP8_E4M3FN && k_rope_scale) return MLA_ERR_UNSUPPORTED_DTYPE;
  return prefill_impl(output, output_dtype, lse, nullptr, nullptr, acc, acc_lse, true,
                      QuerySource{q, nullptr, k_rope, false}, qkv_dtype, k_nope, v, &rows, 0, valid_length,
                      cache_row_offsets, cache_offsets, batch_size, total_q_tokens, num_heads, q_depth, depth, mask,
                      scale, q_scale, k_nope_scale, v_scale, q_max_seq_len, stream);
}

mla_status_t mla_prefill_ragged(void* output, mla_dtype_t output_dtype, const void* q, mla_dtype_t qkv_dtype,
                                const void* k_nope, const void* v, const mla_paged_cache_t* k_rope,
                                uint32_t layer_idx, const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                const uint32_t* cache_offsets, uint32_t batch_size, uint32_t total_q_tokens,
                                uint32_t num_heads, uint32_t q_depth, uint32_t depth, mla_mask_t mask, float scale,
                                const float* q_scale, const float* k_nope_scale, const float* v_scale,
                                uint32_t q_max_seq_len, void* stream) {
  return prefill_impl(output, output_dtype, nullptr, nullptr, nullptr, nullptr, nullptr, false,
                      QuerySource{q, nullptr, nullptr, false}, qkv_dtype, k_nope,
                      v, k_rope, layer_idx, valid_length, cache_row_offsets, cache_offsets, batch_size,
                      total_q_tokens, num_heads, q_depth, depth, mask, scale, q_scale, k_nope_scale, v_scale,
                      q_max_seq_len, stream);
}

mla_status_t mla_prefill_ragged_krope(void* output, mla_dtype_t output_dtype, const void* q, mla_dtype_t qkv_dtype,
                                      const void* k_nope, const void* v, const void* k_rope,
                                      const float* k_rope_scale, const uint32_t* cache_lengths,
                                      const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                      const uint32_t* cache_offsets, uint32_t batch_size, uint32_t total_q_tokens,
                                      uint32_t num_heads, uint32_t q_depth, uint32_t depth, mla_mask_t mask,
                                      float scale, const float* q_scale, const float* k_nope_scale,
                                      const float* v_scale, uint32_t q_max_seq_len, void* stream) {
  if (!k_rope || !cache_lengths) return MLA_ERR_NULL_ARG;
  // the rows' element type is the query's; only the start positions and the
  // rows' scale are taken from this descriptor
  mla_paged_cache_t rows{};
  rows.dtype = qkv_dtype;
  rows.cache_lengths = cache_lengths;
  rows.scale = k_rope_scale;
  if (qkv_dtype != MLA_FP8_E4M3FN && k_rope_scale) return MLA_ERR_UNSUPPORTED_DTYPE;
  return prefill_impl(output, output_dtype, nullptr, nullptr, nullptr, nullptr, nullptr, false,
                      QuerySource{q, nullptr, k_rope, false}, qkv_dtype, k_nope, v, &rows, 0, valid_length,
                      cache_row_offsets, cache_offsets, batch_size, total_q_tokens, num_heads, q_depth, depth, mask,
                      scale, q_scale, k_nope_scale, v_scale, q_max_seq_len, stream);
}

mla_status_t mla_prefill_ragged_kvsplit(void* output, mla_dtype_t output_dtype, float* lse, const void* q,
                                        mla_dtype_t qkv_dtype, const void* k_nope, const void* v,
                                        const mla_paged_cache_t* k_rope, uint32_t layer_idx,
                                        const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                        const uint32_t* cache_offsets, uint32_t batch_size, uint32_t total_q_tokens,
                                        uint32_t num_heads, uint32_t q_depth, uint32_t depth, mla_mask_t mask,
                                        float scale, const float* q_scale, const float* k_nope_scale,
                                        const float* v_scale, uint32_t q_max_seq_len, uint32_t split_keys,
                                        float* workspace, uint64_t workspace_bytes, void* stream) {
  return prefill_impl(output, output_dtype, lse, nullptr, nullptr, nullptr, nullptr, false,
                      QuerySource{q, nullptr, nullptr, false}, qkv_dtype, k_nope, v, k_rope, layer_idx,
                      valid_length, cache_row_offsets, cache_offsets, batch_size, total_q_tokens, num_heads, q_depth,
                      depth, mask, scale, q_scale, k_nope_scale, v_scale, q_max_seq_len, stream,
                      KvSplit{split_keys, workspace, workspace_bytes});
}

mla_status_t mla_prefill_ragged_kvsplit_noalloc(void* output, mla_dtype_t output_dtype, float* lse, const void* q,
                                                mla_dtype_t qkv_dtype, const void* k_nope, const void* v,
                                                const mla_paged_cache_t* k_rope, uint32_t layer_idx,
                                                const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                                const uint32_t* cache_offsets, uint32_t batch_size,
                                                uint32_t total_q_tokens, uint32_t num_heads, uint32_t q_depth,
                                                uint32_t depth, mla_mask_t mask, float scale, const float* q_scale,
                                                const float* k_nope_scale, const float* v_scale,
                                                uint32_t q_max_seq_len, uint32_t split_keys, void* stream) {
  // the partials of a split call must fit the scratch array (checked before the
  // array's address is looked up, so a rejected call touches no GPU)
  if (split_keys != 0 && (split_keys < 128 || mla_prefill_kvsplit_workspace_bytes(total_q_tokens, num_heads) >
                                                  MLA_NOALLOC_SCRATCH_BYTES))
    return MLA_ERR_BAD_SHAPE;
  // an empty call launches nothing and needs no scratch
  const bool split = split_keys != 0 && batch_size != 0 && total_q_tokens != 0 && num_heads != 0;
  float* ws = nullptr;
  if (split) {
    if (g_fail_launch != 0) return hip_status(static_cast<hipError_t>(g_fail_launch));
    const hipError_t e = scratch_of_stream(static_cast<hipStream_t>(stream), &ws);
    if (e != hipSuccess) return hip_status(e);
  }
  // no debug check: it would allocate its flag and synchronise
  return prefill_impl(output, output_dtype, lse, nullptr, nullptr, nullptr, nullptr, false,
                      QuerySource{q, nullptr, nullptr, false}, qkv_dtype, k_nope, v, k_rope, layer_idx,
                      valid_length, cache_row_offsets, cache_offsets, batch_size, total_q_tokens, num_heads, q_depth,
                      depth, mask, scale, q_scale, k_nope_scale, v_scale, q_max_seq_len, stream,
                      KvSplit{split ? split_keys : 0u, ws, MLA_NOALLOC_SCRATCH_BYTES}, false);
}

uint64_t mla_prefill_kvsplit_workspace_bytes(uint32_t total_q_tokens, uint32_t num_heads) {
  // two partial rows of 128 fp32 and two log-sum-exp values per (token, head)
  return (uint64_t)total_q_tokens * num_heads * (2u * 128u + 2u) * sizeof(float);
}

mla_status_t mla_prefill_ragged_split(void* output, mla_dtype_t output_dtype, float* lse, const void* q_nope,
                                      const void* q_rope, mla_dtype_t qkv_dtype, const float* q_scale,
                                      const void* k_nope, const float* k_scales, const void* v,
                                      const float* v_scale, const void* k_rope_rows, const mla_paged_cache_t* kv,
                                      uint32_t layer_idx, const uint32_t* valid_length,
                                      const uint32_t* cache_row_offsets, const uint32_t* cache_offsets,
                                      uint32_t batch_size, uint32_t total_q_tokens, uint32_t num_heads,
                                      uint32_t depth, mla_mask_t mask, float scale, uint32_t q_max_seq_len,
                                      void* stream) {
  return prefill_impl(output, output_dtype, lse, nullptr, nullptr, nullptr, nullptr, false,
                      QuerySource{q_nope, q_rope, k_rope_rows, true}, qkv_dtype, k_nope, v, kv, layer_idx,
                      valid_length, cache_row_offsets, cache_offsets, batch_size, total_q_tokens, num_heads, 128,
                      depth, mask, scale, q_scale, k_scales, v_scale, q_max_seq_len, stream);
}

mla_status_t mla_prefill_latent_up(const mla_paged_cache_t* kv, uint32_t layer_idx, uint32_t batch_size,
                                   const uint32_t* buffer_row_offsets_r, const uint32_t* cache_offsets_r,
                                   uint32_t latent_col, uint32_t latent_dim, const void* w_kv, uint32_t num_heads,
                                   uint32_t buffer_token_size, void* k_nope, void* v, void* stream) {
  mla_status_t st = check_cache(kv, layer_idx);
  if (st != MLA_OK) return st;
  if (!buffer_row_offsets_r || !cache_offsets_r || !w_kv || !k_nope || !v) return MLA_ERR_NULL_ARG;
  if (kv->dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED_DTYPE;
  if (batch_size == 0 || num_heads == 0) return MLA_OK;
  if (batch_size > MLA_MAX_BATCH || buffer_token_size == 0 || latent_dim == 0 || latent_dim % 64 ||
      (uint64_t)latent_col + latent_dim > kv->row_width || (latent_col * 2) % 16 || (kv->row_width * 2) % 16)
    return MLA_ERR_BAD_SHAPE;
  if ((reinterpret_cast<uintptr_t>(kv->data) | reinterpret_cast<uintptr_t>(w_kv) |
       reinterpret_cast<uintptr_t>(k_nope) | reinterpret_cast<uintptr_t>(v)) % 16)
    return MLA_ERR_BAD_SHAPE;
  const uint64_t layer_bytes = (uint64_t)kv->num_pages * kv->page_size * kv->row_width * 2;
  const uint64_t grid = ((uint64_t)buffer_token_size + 127) / 128 * 2 * num_heads;
  if (layer_bytes >= (1ull << 32) || 128ull * latent_dim * 2 >= (1ull << 31) || grid >= (1ull << 31))
    return MLA_ERR_BAD_SHAPE;
  {
    mla::CheckArgs c = check_args(kv, batch_size);
    c.row_offsets = buffer_row_offsets_r;
    c.row_positions = cache_offsets_r;
    c.row_capacity = buffer_token_size;
    st = debug_check(c, stream);
    if (st != MLA_OK) return st;
  }
  mla::LatentArgs a{};
  a.cache = layer_base(kv, layer_idx);
  a.page_table = kv->page_table;
  a.bro = buffer_row_offsets_r;
  a.co = cache_offsets_r;
  a.w = static_cast<const uint16_t*>(w_kv);
  a.k_nope = static_cast<uint16_t*>(k_nope);
  a.v = static_cast<uint16_t*>(v);
  a.max_pages = kv->max_pages_per_seq;
  a.page_size = kv->page_size;
  a.page_shift = (kv->page_size & (kv->page_size - 1)) == 0 ? (uint32_t)__builtin_ctz(kv->page_size) : 0xFFFFFFFFu;
  a.row_bytes = kv->row_width * 2;
  a.latent_col = latent_col;
  a.latent_dim = latent_dim;
  a.cache_bytes = (uint32_t)layer_bytes;
  a.batch = batch_size;
  a.heads = num_heads;
  a.cap = buffer_token_size;
  if (g_fail_launch != 0) return hip_status(static_cast<hipError_t>(g_fail_launch));
  return hip_status(mla::launch_latent_up(a, static_cast<hipStream_t>(stream)));
}

mla_status_t mla_prefill_merge(void* output, mla_dtype_t output_dtype, float* lse, const float* o_a,
                               const float* lse_a, const float* o_b, const float* lse_b, uint32_t total_q_tokens,
                               uint32_t num_heads, uint32_t depth, void* stream) {
  if (!output || !o_a || !lse_a || !o_b || !lse_b) return MLA_ERR_NULL_ARG;
  if (depth != 128) return MLA_ERR_UNSUPPORTED_DIMS;
  if (output_dtype != MLA_BF16 && output_dtype != MLA_FP32) return MLA_ERR_UNSUPPORTED_DTYPE;
  if (total_q_tokens == 0 || num_heads == 0) return MLA_OK;
  if ((reinterpret_cast<uintptr_t>(output) | reinterpret_cast<uintptr_t>(o_a) | reinterpret_cast<uintptr_t>(o_b)) % 16 ||
      (reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(lse_a) | reinterpret_cast<uintptr_t>(lse_b)) % 4)
    return MLA_ERR_BAD_SHAPE;
  const uint64_t rows = (uint64_t)total_q_tokens * num_heads;
  if (rows * 32 / 256 >= (1ull << 31)) return MLA_ERR_BAD_SHAPE;
  mla::MergeArgs a{};
  a.out = output;
  a.lse = lse;
  a.o_a = o_a;
  a.lse_a = lse_a;
  a.o_b = o_b;
  a.lse_b = lse_b;
  a.rows = rows;
  a.out_fp32 = output_dtype == MLA_FP32 ? 1u : 0u;
  if (g_fail_launch != 0) return hip_status(static_cast<hipError_t>(g_fail_launch));
  return hip_status(mla::launch_merge(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
