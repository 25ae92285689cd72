/*
 * mla_prefill.h -- C ABI of the MI355X (gfx950) ragged paged MLA prefill library.
 *
 * Three calls make up one prefill step of a Multi-head Latent Attention layer:
 *
 *   mla_prefill_plan    splits the batch's cached contexts over fixed-capacity
 *                       buffer rows (page "generic_flare_mla_prefill_ragged_paged_plan");
 *   mla_prefill_gather  copies one buffer row's cache entries out of the paged
 *                       cache into a contiguous buffer (same page, description: the
 *                       plan exists so that K/V entries can be gathered);
 *   mla_prefill_ragged  masked (causal or null) attention of ragged Q [T,H,192]
 *                       over the ragged K_nope/V buffer [rows,H,128] and the
 *                       shared, paged K_rope [positions,1,64] (page
 *                       "flare_mla_prefill"; launch shape and argument meanings
 *                       of page "mla_prefill_v2_ragged").
 *
 * The other calls widen that step:
 *
 *   mla_prefill_ragged_split  the same attention for a query given in two parts,
 *                       q_nope and q_rope, and K_rope from the cache or from
 *                       contiguous rows (page "flare_mla_prefill", the q_nope /
 *                       q_rope / q_scale / k_scales overloads).
 *
 *   mla_prefill_ragged_krope  the same attention with K_rope given as rows laid
 *                       out like K (what mla_prefill_gather makes of the cache's
 *                       K_rope column window).
 *
 *   mla_prefill_latent_up  per-head K_nope / V of one buffer row, up-projected
 *                       from the latent part of the cache rows the plan row holds.
 *
 *   mla_prefill_ragged_kvsplit  the attention of mla_prefill_ragged with the
 *                       key range of long query tiles split over two workgroups
 *                       and merged (for grids with few tiles, e.g. few heads).
 *
 *   mla_prefill_check   tests on the device the preconditions the calls document
 *                       but do not check (offsets, positions, page ids);
 *                       mla_prefill_set_debug makes every call run it first.
 *
 * When the plan cuts the contexts over several buffer rows, each row's
 * attention covers part of a sequence's keys:
 *
 *   mla_prefill_ragged_lse  the same attention, also writing each (token, head)'s
 *                           log-sum-exp, optionally merged in place with the
 *                           partial result of earlier rows;
 *   mla_prefill_ragged_row  one row of such a plan, rows run in order: each
 *                           token's partial is carried in an fp32 accumulator
 *                           from its sequence's first row to the row holding its
 *                           last visible key, which writes the output;
 *   mla_prefill_ragged_row_krope  the same with K_rope as the row's gathered rows;
 *   mla_prefill_merge       log-sum-exp combine of two partial results.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked [host].  Device arrays are
 *     dense and row-major in the shapes given; element types are exact.
 *   - Every call only validates its host-side arguments and enqueues work on
 *     `stream` (a hipStream_t passed as void*; NULL = the null stream); it never
 *     synchronises.  The caller owns all memory and keeps it alive and unchanged
 *     until the enqueued work has finished.  The library allocates no device
 *     memory and keeps no state beyond its loaded code objects (debug mode
 *     aside: its on/off setting and one 4-byte flag per GPU); calls are
 *     thread-safe.  Outputs must not alias inputs, except where a call says so.
 *   - Host-checkable errors are returned before anything is enqueued (nothing
 *     is written).  Properties of device data (monotone offsets, in-range page
 *     ids, lengths) are preconditions that are NOT checked: violating them is
 *     undefined behaviour; mla_prefill_check tests them on the device, and in
 *     debug mode (mla_prefill_set_debug, or MLA_PREFILL_DEBUG=1 in the
 *     environment when the library loads) every call runs that check first,
 *     synchronises and returns MLA_ERR_PRECONDITION instead of launching on
 *     violating data.  MLA_ERR_HIP reports a failed launch
 *     (hipGetLastError after the enqueue); mla_prefill_last_hip_error() then
 *     returns the HIP error code.
 *   - batch_size == 0 (or total_q_tokens == 0 for the attention) is a valid no-op.
 */
#ifndef MLA_PREFILL_H
#define MLA_PREFILL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_ARG = 1,          /* a required pointer is NULL */
  MLA_ERR_BAD_SHAPE = 2,         /* sizes are inconsistent or out of the supported range */
  MLA_ERR_UNSUPPORTED_DTYPE = 3, /* dtype combination not offered */
  MLA_ERR_UNSUPPORTED_DIMS = 4,  /* q_depth != 192 or depth != 128 */
  MLA_ERR_UNSUPPORTED_MASK = 5,  /* mask kind not offered */
  MLA_ERR_HIP = 6,               /* the HIP runtime reported an error on enqueue */
  MLA_ERR_PRECONDITION = 7       /* debug mode only: the device data violate a documented
                                    precondition (see mla_prefill_check); nothing was launched */
} mla_status_t;

/* Element types ("flare_mla_prefill", Parameters: q is bfloat16 or float8_e4m3fn;
 * the output is bfloat16 when q is float8_e4m3fn, else the type of q).
 * MLA_FP32 is offered for outputs only: partial results that are merged later
 * keep full precision. */
typedef enum { MLA_BF16 = 0, MLA_FP8_E4M3FN = 1, MLA_FP32 = 2 } mla_dtype_t;

/* Mask predicates ("mla_prefill_v2_ragged", Parameters and Args: mask_t and
 * mask_functor, "causal, null, etc."):
 *   MLA_MASK_CAUSAL  key position kpos is visible to query position qpos iff kpos <= qpos;
 *   MLA_MASK_NULL    no predicate: every key the call is given for sequence b is
 *                    visible to every new token of b. */
typedef enum { MLA_MASK_CAUSAL = 0, MLA_MASK_NULL = 1 } mla_mask_t;

/* Largest batch the plan and gather kernels accept (their per-sequence offsets
 * are staged in on-chip memory). */
#define MLA_MAX_BATCH 8192

/*
 * One layer-indexed paged KV cache ("generic_flare_mla_prefill_ragged_paged_plan",
 * Args: kv_collection and layer_idx).  The struct itself is [host]; it is read
 * during the call only.
 *
 *   data          device, [num_layers][num_pages][page_size][1][row_width]
 *                 elements of `dtype` (one KV head per cache row).
 *   page_table    device uint32 [batch_size][max_pages_per_seq]: cache position
 *                 pos of sequence b lives in physical page
 *                 page_table[b][pos / page_size], slot pos % page_size.
 *   cache_lengths device uint32 [batch_size]: tokens of sequence b cached before
 *                 this step (its start position; "mla_prefill_v2_ragged", Args:
 *                 k_nope).  Positions [0, cache_lengths[b] + n_b) are in the cache
 *                 when the step runs, n_b being the step's new tokens.
 *   rope_col      first of the 64 columns holding K_rope in a cache row
 *                 ("flare_mla_prefill", Args: k_rope); rope_col + 64 <= row_width.
 *   scale         device fp32 scalar, the per-tensor dequantisation scale of an
 *                 MLA_FP8_E4M3FN cache; ignored (may be NULL) for MLA_BF16.
 */
typedef struct {
  const void* data;
  mla_dtype_t dtype;
  uint32_t num_layers;
  uint32_t num_pages;
  uint32_t page_size;
  uint32_t row_width;
  uint32_t rope_col;
  const uint32_t* page_table;
  uint32_t max_pages_per_seq;
  const uint32_t* cache_lengths;
  const float* scale;
} mla_paged_cache_t;

/*
 * mla_prefill_plan -- page "generic_flare_mla_prefill_ragged_paged_plan",
 * description and Args.
 *
 * Sequence b has n_b = input_row_offsets[b+1] - input_row_offsets[b] new tokens
 * and a context of L_b = kv->cache_lengths[b] + n_b cache positions.  The
 * contexts are laid end to end in batch order (S_b = L_0 + ... + L_{b-1},
 * C = S_B) and cut into rows of `buffer_token_size` tokens; a sequence may
 * straddle rows.  For each row r < min(num_buffer_rows, ceil(C / cap)):
 *   buffer_row_offsets[r][b] = clamp(S_b - r*cap, 0, cap)        (b = 0..B)
 *   cache_offsets[r][b]      = clamp(r*cap - S_b, 0, L_b)         (b < B)
 *   buffer_lengths[r]        = buffer_row_offsets[r][B]
 * so row r holds sequence b's cache positions [cache_offsets[r][b], +len) at
 * buffer slots [buffer_row_offsets[r][b], buffer_row_offsets[r][b+1]).  Rows the
 * batch does not reach get zero offsets and buffer_lengths[r] = -1.
 *
 *   input_row_offsets   device uint32 [batch_size+1], non-decreasing, [0] = 0.
 *   kv                  [host] cache descriptor; only cache_lengths is read.
 *   layer_idx           < kv->num_layers.
 *   buffer_token_size   cap > 0.
 *   num_buffer_rows     R >= 1, the rows the outputs are sized for.
 *   buffer_row_offsets  device uint32 [R][batch_size+1] (output).
 *   cache_offsets       device uint32 [R][batch_size] (output).
 *   buffer_lengths      device int32 [R] (output).
 *   device_status       device int32 scalar or NULL (output): 1 when R rows
 *                       cannot hold the batch (R*cap < C), else 0.
 * Errors: NULL_ARG; BAD_SHAPE for cap == 0, R == 0, layer_idx out of range or
 * batch_size > MLA_MAX_BATCH.  Exact integer arithmetic (64-bit internally).
 */
mla_status_t mla_prefill_plan(const uint32_t* input_row_offsets, uint32_t batch_size,
                              const mla_paged_cache_t* kv, uint32_t layer_idx,
                              uint32_t buffer_token_size, uint32_t num_buffer_rows,
                              uint32_t* buffer_row_offsets, uint32_t* cache_offsets,
                              int32_t* buffer_lengths, int32_t* device_status, void* stream);

/*
 * mla_prefill_gather -- copies one plan row's cache entries into a contiguous
 * buffer (page "generic_flare_mla_prefill_ragged_paged_plan", description).
 *
 * For every b < batch_size and j < buffer_row_offsets_r[b+1] - buffer_row_offsets_r[b]:
 *   out[buffer_row_offsets_r[b] + j][c] = cache row of sequence b at position
 *   cache_offsets_r[b] + j, column col_begin + c, for c < col_count.
 * Slots at or beyond buffer_row_offsets_r[batch_size] are left untouched.  A
 * byte-exact copy in kv->dtype.
 *
 *   buffer_row_offsets_r  device uint32 [batch_size+1]: one row of the plan output.
 *   cache_offsets_r       device uint32 [batch_size]: the same row's cache offsets.
 *   col_begin, col_count  column window, col_begin + col_count <= kv->row_width, col_count >= 1.
 *   buffer_token_size     rows of `out` (the plan's cap); buffer_row_offsets_r[B] <= it.
 *   out                   device [buffer_token_size][col_count] elements of kv->dtype.
 * Errors: NULL_ARG, BAD_SHAPE (column window, layer, batch_size > MLA_MAX_BATCH).
 */
mla_status_t mla_prefill_gather(const mla_paged_cache_t* kv, uint32_t layer_idx, uint32_t batch_size,
                                const uint32_t* buffer_row_offsets_r, const uint32_t* cache_offsets_r,
                                uint32_t col_begin, uint32_t col_count, uint32_t buffer_token_size,
                                void* out, void* stream);

/*
 * mla_prefill_latent_up -- the K_nope / V buffer of one plan row, decompressed
 * from the latent cache.  The pages describe the cache as a latent cache (page
 * "mla_prefill_v2_ragged", Args: V is the nope segment of the latent cache)
 * and the plan that says which cache positions fill which buffer slots (page
 * "generic_flare_mla_prefill_ragged_paged_plan"); the decompression is the
 * DeepSeek-V2/V3 one.  For every b < batch_size, j < bro[b+1] - bro[b], slot
 * g = bro[b] + j and head h:
 *   c_g              = cache row of sequence b at position co[b] + j, columns
 *                      latent_col .. latent_col + latent_dim - 1 (as mla_prefill_gather)
 *   k_nope[g][h][d]  = sum_c w_kv[h*256 + d][c]       * c_g[c]     (d < 128)
 *   v[g][h][d]       = sum_c w_kv[h*256 + 128 + d][c] * c_g[c]
 * accumulated in fp32 and rounded to bf16 (nearest-even).  Slots at or beyond
 * bro[batch_size] are not written.
 *
 *   kv                   [host] bf16 cache descriptor (page table, rows).
 *   buffer_row_offsets_r, cache_offsets_r  one plan row, as for mla_prefill_gather.
 *   latent_col, latent_dim  latent column window; latent_dim a positive multiple
 *                        of 64, latent_col * 2 bytes a multiple of 16.
 *   w_kv                 device bf16 [num_heads * 256][latent_dim]: per head 128
 *                        key rows then 128 value rows (a linear layer's weight,
 *                        output features by input features).
 *   buffer_token_size    slots of k_nope / v (the plan's cap).
 *   k_nope, v            device bf16 [buffer_token_size][num_heads][128] (outputs),
 *                        16-byte aligned.
 * Errors: NULL_ARG, UNSUPPORTED_DTYPE (cache not bf16), BAD_SHAPE (window,
 * alignment, batch_size > MLA_MAX_BATCH, sizes past 32-bit offsets), HIP.
 */
mla_status_t mla_prefill_latent_up(const mla_paged_cache_t* kv, uint32_t layer_idx, uint32_t batch_size,
                                   const uint32_t* buffer_row_offsets_r, const uint32_t* cache_offsets_r,
                                   uint32_t latent_col, uint32_t latent_dim, const void* w_kv,
                                   uint32_t num_heads, uint32_t buffer_token_size, void* k_nope, void* v,
                                   void* stream);

/*
 * mla_prefill_ragged -- page "flare_mla_prefill" (description, Args) with the
 * paged k_rope operand; launch semantics of page "mla_prefill_v2_ragged".
 *
 * Sequence b owns query tokens t = valid_length[b] + i, i < n_b = valid_length[b+1]
 * - valid_length[b], at cache positions qpos = kv->cache_lengths[b] + i, and keys
 * g = cache_row_offsets[b] + j, j < cache_row_offsets[b+1] - cache_row_offsets[b],
 * at cache positions kpos = cache_offsets[b] + j (0 + j when cache_offsets is
 * NULL: a contiguous cache).  For every t and head h:
 *   s_j = scale * ( sum_{d<128} q[t][h][d] * k_nope[g][h][d]
 *                 + sum_{e<64}  q[t][h][128+e] * K_rope(b, kpos)[e] )
 *   output[t][h][:] = sum_{j visible} softmax_j(s) * v[g][h][:]
 * where K_rope(b, pos) is the 64-wide column window at kv->rope_col of the cache
 * row of sequence b at position pos in layer layer_idx (one row shared by all
 * heads), "visible" means kpos <= qpos under MLA_MASK_CAUSAL and every j under
 * MLA_MASK_NULL, and a query with no visible key gets 0.
 *
 *   output            device [total_q_tokens][num_heads][128], output_dtype.
 *   q                 device [total_q_tokens][num_heads][192], qkv_dtype
 *                     (columns 0..127 pair with k_nope, 128..191 with K_rope).
 *   k_nope, v         device [rows][num_heads][128], qkv_dtype, rows >=
 *                     cache_row_offsets[batch_size].
 *   k_rope            [host] paged cache descriptor; kv->dtype must be qkv_dtype.
 *   valid_length      device uint32 [batch_size+1], ragged Q offsets,
 *                     valid_length[batch_size] == total_q_tokens.
 *   cache_row_offsets device uint32 [batch_size+1], ragged K/V offsets.
 *   cache_offsets     device uint32 [batch_size] or NULL.
 *   q_depth, depth    must be 192 and 128 (DeepSeek V2/V3 geometry).
 *   scale             [host] softmax scale multiplying q.k; any sign, zero
 *                     allowed.  The weights are formed in fp32 as
 *                     exp2(s * c - m * c), c = |scale| * log2(e), m a running
 *                     score: the rounding of m * c puts an absolute error of
 *                     about 1e-7 * |scale * q.k| into each exponent, below the
 *                     bf16 rounding of the weights while |scale * q.k| < 3e4.
 *                     Larger products still give one-hot softmaxes exactly (the
 *                     GPU tests go to |scale| = 1e4 on unit-variance inputs);
 *                     |scale| above about 1e8 is outside the fp32 range of the
 *                     formulation and not supported.
 *   q_scale, k_nope_scale, v_scale
 *                     fp8 only: device fp32 per-tensor dequantisation scales
 *                     (K_rope uses kv->scale); must be NULL for bf16.
 *   q_max_seq_len     upper bound on n_b (bounds the launch); 0 = total_q_tokens.
 *                     A value below some n_b is a precondition violation.
 *   mask              MLA_MASK_CAUSAL or MLA_MASK_NULL.
 * Dtypes: qkv MLA_BF16 or MLA_FP8_E4M3FN; output MLA_BF16 (the pages' type) or
 * MLA_FP32.  Accumulation is fp32; a bf16 output is rounded to nearest-even.
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED_DTYPE, UNSUPPORTED_DIMS,
 * UNSUPPORTED_MASK, HIP.
 */
mla_status_t mla_prefill_ragged(void* output, mla_dtype_t output_dtype, const void* q, mla_dtype_t qkv_dtype,
                                const void* k_nope, const void* v, const mla_paged_cache_t* k_rope,
                                uint32_t layer_idx, const uint32_t* valid_length,
                                const uint32_t* cache_row_offsets, const uint32_t* cache_offsets,
                                uint32_t batch_size, uint32_t total_q_tokens, uint32_t num_heads,
                                uint32_t q_depth, uint32_t depth, mla_mask_t mask, float scale,
                                const float* q_scale, const float* k_nope_scale, const float* v_scale,
                                uint32_t q_max_seq_len, void* stream);

/*
 * mla_prefill_ragged_krope -- page "flare_mla_prefill", the overload whose
 * k_rope is a tensor rather than the paged cache; the plan of page
 * "generic_flare_mla_prefill_ragged_paged_plan" exists so that the K/V entries
 * of a buffer row can be gathered into contiguous rows, which mla_prefill_gather
 * does for the K_rope column window.
 *
 * The attention of mla_prefill_ragged with K_rope(b, kpos) = k_rope row
 * cache_row_offsets[b] + j (the row laid out like k_nope's key j of sequence
 * b) instead of a cache read; start positions are cache_lengths[b].
 *
 *   k_rope          device [rows][1][64], qkv_dtype, 16-byte aligned; fp8 values
 *                   stand for code * (*k_rope_scale).
 *   k_rope_scale    device fp32 scalar: required for MLA_FP8_E4M3FN, NULL for bf16.
 *   cache_lengths   device uint32 [batch_size], start position p_b of each sequence.
 * All other arguments as mla_prefill_ragged.
 * Errors: as mla_prefill_ragged.
 */
mla_status_t mla_prefill_ragged_krope(void* output, mla_dtype_t output_dtype, const void* q, mla_dtype_t qkv_dtype,
                                      const void* k_nope, const void* v, const void* k_rope,
                                      const float* k_rope_scale, const uint32_t* cache_lengths,
                                      const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                      const uint32_t* cache_offsets, uint32_t batch_size, uint32_t total_q_tokens,
                                      uint32_t num_heads, uint32_t q_depth, uint32_t depth, mla_mask_t mask,
                                      float scale, const float* q_scale, const float* k_nope_scale,
                                      const float* v_scale, uint32_t q_max_seq_len, void* stream);

/*
 * mla_prefill_ragged_lse -- the attention of mla_prefill_ragged for one buffer
 * row of the plan (page "generic_flare_mla_prefill_ragged_paged_plan",
 * description and Args: a row holds part of each sequence's cached context),
 * with the log-sum-exp a later merge needs.
 *
 * All arguments from q on are those of mla_prefill_ragged, with the same
 * meaning and checks.  For every token t and head h the call computes the
 * softmax result o over the keys it is given, as mla_prefill_ragged does, and
 *   lse_self[t][h] = ln( sum_{j visible} exp(s_j) )        (-inf: no visible key)
 * with s_j the scaled scores above.  Then:
 *   prev_output == NULL:  output = o, lse = lse_self;
 *   otherwise (a partial over other keys of the same tokens), the softmax over
 *   the union:  L = ln(exp(prev_lse) + exp(lse_self)),
 *               output = exp(prev_lse - L) * prev_output + exp(lse_self - L) * o,
 *               lse = L   (both -inf: output 0, lse -inf).
 * Running the call once per buffer row, passing the previous call's fp32
 * output and lse as prev_*, therefore yields the attention over every key.
 *
 *   output        device [total_q_tokens][num_heads][128], MLA_BF16 or MLA_FP32.
 *   lse           device fp32 [total_q_tokens][num_heads] or NULL (not written).
 *   prev_output   device fp32 [total_q_tokens][num_heads][128] or NULL; may be
 *                 the same buffer as `output` when output_dtype is MLA_FP32.
 *   prev_lse      device fp32 [total_q_tokens][num_heads]; NULL exactly when
 *                 prev_output is; may be the same buffer as `lse`.
 * Every (t, h) with t < total_q_tokens inside some sequence is written on every
 * call, also where this call sees no key (it then passes prev_* through).
 * prev_output is not read where its weight is 0 (prev_lse = -inf).
 * Errors: those of mla_prefill_ragged; NULL_ARG when exactly one of prev_output
 * and prev_lse is NULL; BAD_SHAPE for fp32 arrays not 4-byte (lse) or 16-byte
 * (prev_output) aligned.
 */
mla_status_t mla_prefill_ragged_lse(void* output, mla_dtype_t output_dtype, float* lse,
                                    const float* prev_output, const float* prev_lse,
                                    const void* q, mla_dtype_t qkv_dtype, const void* k_nope, const void* v,
                                    const mla_paged_cache_t* k_rope, uint32_t layer_idx,
                                    const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                    const uint32_t* cache_offsets, uint32_t batch_size,
                                    uint32_t total_q_tokens, uint32_t num_heads, uint32_t q_depth,
                                    uint32_t depth, mla_mask_t mask, float scale, const float* q_scale,
                                    const float* k_nope_scale, const float* v_scale,
                                    uint32_t q_max_seq_len, void* stream);

/*
 * mla_prefill_ragged_split -- page "flare_mla_prefill", the overloads whose query
 * is split into q_nope (element type `dtype`, with q_scale) and q_rope, whose K
 * carries k_scales, and whose k_rope is either the paged cache or a plain tensor.
 *
 * The attention of mla_prefill_ragged with q[t][h][0..127] = q_nope[t][h][:] and
 * q[t][h][128..191] = q_rope[t][h][:], where:
 *   q_nope        device [total_q_tokens][num_heads][128], qkv_dtype; fp8 values
 *                 stand for code * (*q_scale).
 *   q_rope        device [total_q_tokens][num_heads][64], bf16, never scaled.
 *   k_nope, v     device [rows][num_heads][128], qkv_dtype; fp8: code * (*k_scales)
 *                 and code * (*v_scale) (one fp32 per tensor).
 *   k_rope_rows   contiguous K_rope, device [rows][1][64] laid out like k_nope:
 *                 key j of sequence b uses row cache_row_offsets[b] + j (each
 *                 64-key tile is addressed from its own first row, so a
 *                 sequence's rows may span more than 4 GiB).  Their element
 *                 type is kv->dtype: bf16, or e4m3 (qkv_dtype MLA_FP8_E4M3FN
 *                 only) standing for code * (*kv->scale), converted exactly to
 *                 bf16 for its product with q_rope.  NULL:
 *                 K_rope comes from the paged cache `kv` as in mla_prefill_ragged
 *                 (a bf16 cache, or an e4m3 cache with kv->scale when qkv_dtype is
 *                 MLA_FP8_E4M3FN; e4m3 K_rope is converted exactly to bf16 for its
 *                 product with q_rope).
 *   kv            [host] cache descriptor.  With k_rope_rows only kv->cache_lengths
 *                 (the start positions), kv->dtype and kv->scale (the rows'
 *                 element type and scale) are read.
 *   q_scale, k_scales, v_scale  device fp32 scalars, required for MLA_FP8_E4M3FN
 *                 and NULL for MLA_BF16.
 * Other arguments as in mla_prefill_ragged; depth must be 128.  output is bf16
 * or fp32; lse (fp32 [total_q_tokens][num_heads] or NULL) receives each (token,
 * head)'s log-sum-exp as in mla_prefill_ragged_lse.  The score is
 *   s_j = scale * ( q_nope . k_nope + q_rope . K_rope )  on the dequantised values.
 * Errors: NULL_ARG (q_rope, required scales, kv->cache_lengths), BAD_SHAPE
 * (16-byte alignment of q_nope, q_rope, k_rope_rows, k_nope, v, output),
 * UNSUPPORTED_DTYPE (bf16 q_nope with an e4m3 cache, scales given for bf16),
 * UNSUPPORTED_DIMS, UNSUPPORTED_MASK, HIP.
 */
mla_status_t mla_prefill_ragged_split(void* output, mla_dtype_t output_dtype, float* lse, const void* q_nope,
                                      const void* q_rope, mla_dtype_t qkv_dtype, const float* q_scale,
                                      const void* k_nope, const float* k_scales, const void* v,
                                      const float* v_scale, const void* k_rope_rows, const mla_paged_cache_t* kv,
                                      uint32_t layer_idx, const uint32_t* valid_length,
                                      const uint32_t* cache_row_offsets, const uint32_t* cache_offsets,
                                      uint32_t batch_size, uint32_t total_q_tokens, uint32_t num_heads,
                                      uint32_t depth, mla_mask_t mask, float scale, uint32_t q_max_seq_len,
                                      void* stream);

/*
 * mla_prefill_ragged_kvsplit -- the attention of mla_prefill_ragged (page
 * "flare_mla_prefill", description and Args), with the log-sum-exp of
 * mla_prefill_ragged_lse, scheduled for batches with few query tiles per head
 * count (for instance one GPU's share of the heads under tensor parallelism).
 * The pages fix what is computed, not how the work is cut; this call cuts it by
 * the split-KV scheme published as Flash-Decoding (Dao, Haziza, Massa, Sizov,
 * 2023): a 128-query tile of one sequence and head whose visible keys number
 * more than split_keys is computed by two workgroups, one per half of its
 * 64-key tiles, each writing its normalised fp32 partial and log-sum-exp to
 * `workspace`; a second kernel on the same stream combines the two as
 * mla_prefill_merge does.  Other tiles are computed whole, as in
 * mla_prefill_ragged.  The result equals mla_prefill_ragged's up to fp32
 * rounding order (the partials are fp32; a bf16 output is rounded once, after
 * the combine).
 *
 * All arguments up to q_max_seq_len are those of mla_prefill_ragged_lse
 * without prev_output / prev_lse, with the same meaning and checks; lse may
 * be NULL.
 *   split_keys       [host] 0: no tile is split (workspace is not used); else
 *                    at least 128.  A smaller value splits more tiles.
 *   workspace        device fp32, 16-byte aligned, at least
 *                    mla_prefill_kvsplit_workspace_bytes(total_q_tokens,
 *                    num_heads) bytes; owned by the caller, contents on entry
 *                    ignored, contents on exit unspecified; must not overlap
 *                    any other argument.  May be NULL when split_keys is 0.
 *   workspace_bytes  [host] its size in bytes.
 * Two calls that share a workspace must be ordered (one stream, or events).
 * Errors: those of mla_prefill_ragged_lse; NULL_ARG for a NULL workspace with
 * split_keys > 0; BAD_SHAPE for split_keys in 1..127, a workspace that is too
 * small or not 16-byte aligned.
 */
mla_status_t mla_prefill_ragged_kvsplit(void* output, mla_dtype_t output_dtype, float* lse, const void* q,
                                        mla_dtype_t qkv_dtype, const void* k_nope, const void* v,
                                        const mla_paged_cache_t* k_rope, uint32_t layer_idx,
                                        const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                        const uint32_t* cache_offsets, uint32_t batch_size,
                                        uint32_t total_q_tokens, uint32_t num_heads, uint32_t q_depth,
                                        uint32_t depth, mla_mask_t mask, float scale, const float* q_scale,
                                        const float* k_nope_scale, const float* v_scale, uint32_t q_max_seq_len,
                                        uint32_t split_keys, float* workspace, uint64_t workspace_bytes,
                                        void* stream);

/* Workspace bytes mla_prefill_ragged_kvsplit needs: total_q_tokens * num_heads
 * * (2 * 128 + 2) * 4 (two fp32 partial rows and two log-sum-exp values per
 * token and head). */
uint64_t mla_prefill_kvsplit_workspace_bytes(uint32_t total_q_tokens, uint32_t num_heads);

/* Bytes of the scratch array of mla_prefill_ragged_kvsplit_noalloc (64 MiB):
 * split calls with mla_prefill_kvsplit_workspace_bytes(total_q_tokens,
 * num_heads) up to this size, i.e. total_q_tokens * num_heads <= 65,027. */
#define MLA_NOALLOC_SCRATCH_BYTES (64ull << 20)

/*
 * mla_prefill_ragged_kvsplit_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): mla_prefill_ragged_kvsplit without the workspace
 * arguments.  The key split's partial rows and log-sum-exps go to a device array
 * of the library (MLA_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the
 * process ends; its address is looked up once per GPU, on the first split call
 * there).  The call allocates nothing and calls no allocating routine; debug
 * mode does not apply to it.  Nothing in the array has to start at zero (each
 * split tile's two halves write their partials before the merge reads them).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: two split calls whose work may overlap in time on one GPU (other
 * streams, or graphs replayed concurrently) race and must not be issued.
 * Outputs are those of mla_prefill_ragged_kvsplit with the same split_keys.
 * Errors: as mla_prefill_ragged_kvsplit; BAD_SHAPE also for a split call
 * (split_keys != 0) whose partials exceed MLA_NOALLOC_SCRATCH_BYTES.
 */
mla_status_t mla_prefill_ragged_kvsplit_noalloc(void* output, mla_dtype_t output_dtype, float* lse, const void* q,
                                                mla_dtype_t qkv_dtype, const void* k_nope, const void* v,
                                                const mla_paged_cache_t* k_rope, uint32_t layer_idx,
                                                const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                                const uint32_t* cache_offsets, uint32_t batch_size,
                                                uint32_t total_q_tokens, uint32_t num_heads, uint32_t q_depth,
                                                uint32_t depth, mla_mask_t mask, float scale, const float* q_scale,
                                                const float* k_nope_scale, const float* v_scale,
                                                uint32_t q_max_seq_len, uint32_t split_keys, void* stream);

/*
 * mla_prefill_ragged_row -- one buffer row of the plan of page
 * "generic_flare_mla_prefill_ragged_paged_plan" (description, Args: rows of
 * fixed capacity, each sequence's slice given by its buffer_row_offsets and
 * cache_offsets), when the plan cut the batch's contexts over several rows.
 *
 * All arguments from q on are those of mla_prefill_ragged, with the same
 * meaning and checks; cache_row_offsets / cache_offsets must be row r of the
 * plan (its buffer_row_offsets[r] and cache_offsets[r]) and k_nope / v that
 * row's K/V buffer.  The call is made once per row, r = 0, 1, ..., in order on
 * one stream, with the same acc / acc_lse for every row of the batch.  For a
 * query token i of sequence b whose slice in this row is not empty, with len_b
 * keys starting at cache position c_b = cache_offsets[b], and k_i the cache
 * position of the token's last visible key (p_b + i under the causal mask,
 * p_b + n_b - 1 under the null mask; p_b = kv->cache_lengths[b]):
 *   k_i < c_b                       the row holds none of its keys: not touched;
 *   c_b == 0 (first row), k_i >= len_b
 *                                   the row's partial (output and lse as in
 *                                   mla_prefill_ragged_lse) goes to acc / acc_lse;
 *   c_b > 0, k_i >= c_b + len_b     the row's partial is merged into acc / acc_lse;
 *   c_b > 0, c_b <= k_i < c_b + len_b (the row holding its last key)
 *                                   the row's partial is merged with acc / acc_lse
 *                                   and the result goes to output (and lse);
 *   c_b == 0, k_i < len_b           the row's result goes straight to output (and lse).
 * So each token is finished by the row holding its last visible key, and later
 * rows leave it alone (under the causal mask the tokens of a sequence finish in
 * different rows).  acc / acc_lse hold no defined values for finished tokens.
 * After the last row, output holds the attention over every key of every
 * sequence (what mla_prefill_ragged computes over one row holding all of them),
 * and lse, when given, its log-sum-exp.
 *
 *   output      device [total_q_tokens][num_heads][128], MLA_BF16 or MLA_FP32.
 *   lse         device fp32 [total_q_tokens][num_heads] or NULL.
 *   acc         device fp32 [total_q_tokens][num_heads][128], 16-byte aligned;
 *               acc_lse device fp32 [total_q_tokens][num_heads].  Scratch owned by
 *               the caller, carried between the rows of one batch; no initial
 *               contents are needed.
 * Errors: those of mla_prefill_ragged; NULL_ARG when acc or acc_lse is NULL.
 */
mla_status_t mla_prefill_ragged_row(void* output, mla_dtype_t output_dtype, float* lse, float* acc,
                                    float* acc_lse, const void* q, mla_dtype_t qkv_dtype, const void* k_nope,
                                    const void* v, const mla_paged_cache_t* k_rope, uint32_t layer_idx,
                                    const uint32_t* valid_length, const uint32_t* cache_row_offsets,
                                    const uint32_t* cache_offsets, uint32_t batch_size,
                                    uint32_t total_q_tokens, uint32_t num_heads, uint32_t q_depth,
                                    uint32_t depth, mla_mask_t mask, float scale, const float* q_scale,
                                    const float* k_nope_scale, const float* v_scale,
                                    uint32_t q_max_seq_len, void* stream);

/*
 * mla_prefill_ragged_row_krope -- mla_prefill_ragged_row with K_rope given as
 * rows laid out like K (page "flare_mla_prefill", the overload whose k_rope is
 * a tensor): for a row of the plan whose K_rope window has been gathered into
 * contiguous rows (mla_prefill_gather of columns [rope_col, rope_col + 64)),
 * so that the gather feeds the attention of every row of a multi-row plan.
 *
 *   k_rope, k_rope_scale, cache_lengths   as mla_prefill_ragged_krope: k_rope
 *                   row cache_row_offsets[b] + j holds key j of sequence b's
 *                   slice in this row.
 * All other arguments, the per-token rule for acc / acc_lse / output, and the
 * errors as mla_prefill_ragged_row.  The arithmetic is that call's, so with rows
 * holding what the page table points at the outputs are the same bit for bit.
 */
mla_status_t mla_prefill_ragged_row_krope(void* output, mla_dtype_t output_dtype, float* lse, float* acc,
                                          float* acc_lse, const void* q, mla_dtype_t qkv_dtype, const void* k_nope,
                                          const void* v, const void* k_rope, const float* k_rope_scale,
                                          const uint32_t* cache_lengths, const uint32_t* valid_length,
                                          const uint32_t* cache_row_offsets, const uint32_t* cache_offsets,
                                          uint32_t batch_size, uint32_t total_q_tokens, uint32_t num_heads,
                                          uint32_t q_depth, uint32_t depth, mla_mask_t mask, float scale,
                                          const float* q_scale, const float* k_nope_scale, const float* v_scale,
                                          uint32_t q_max_seq_len, void* stream);

/*
 * mla_prefill_merge -- combine two partial attention results over disjoint key
 * sets of the same tokens (buffer rows of page
 * "generic_flare_mla_prefill_ragged_paged_plan"; see mla_prefill_ragged_lse).
 * For every row r < total_q_tokens * num_heads:
 *   L = ln(exp(lse_a[r]) + exp(lse_b[r])),
 *   output[r][:] = exp(lse_a[r] - L) * o_a[r][:] + exp(lse_b[r] - L) * o_b[r][:],
 *   lse[r] = L          (lse_a = lse_b = -inf: output 0, lse -inf).
 * A side whose weight is 0 is not read.
 *
 *   output      device [total_q_tokens][num_heads][depth], MLA_BF16 or MLA_FP32;
 *               may be o_a or o_b when MLA_FP32.
 *   lse         device fp32 [total_q_tokens][num_heads] or NULL; may be lse_a or lse_b.
 *   o_a, o_b    device fp32 [total_q_tokens][num_heads][depth].
 *   lse_a, lse_b device fp32 [total_q_tokens][num_heads] (natural log).
 *   depth       must be 128.
 * Errors: NULL_ARG, UNSUPPORTED_DIMS, UNSUPPORTED_DTYPE, BAD_SHAPE (alignment:
 * 16 bytes for output, o_a, o_b; 4 for the lse arrays), HIP.
 */
mla_status_t mla_prefill_merge(void* output, mla_dtype_t output_dtype, float* lse, const float* o_a,
                               const float* lse_a, const float* o_b, const float* lse_b,
                               uint32_t total_q_tokens, uint32_t num_heads, uint32_t depth, void* stream);

/*
 * mla_prefill_check -- tests on the device the preconditions of the plan,
 * gather, attention and decompression calls that the host cannot see (their
 * documented "not checked" device data: page "generic_flare_mla_prefill_ragged_paged_plan",
 * Args, and page "flare_mla_prefill", Args, for the meaning of each array), and
 * ORs the bits of every violated one into *violations.  It reads the arrays
 * only inside their documented extents (page-table reads are clamped to the
 * sequence's row of max_pages_per_seq entries) and never uses a value it
 * checks as an address, so it is safe on any data.
 *
 *   kv              [host] cache descriptor: cache_lengths (device [B]) is
 *                   required; page_table may be NULL (no paged reads to check,
 *                   e.g. contiguous K_rope rows), else page_size,
 *                   max_pages_per_seq and num_pages must be > 0.
 *   valid_length    device [B+1] new-token offsets, or NULL (not checked).
 *   total_q_tokens  checked against valid_length[B] unless it is 0xFFFFFFFF.
 *   q_max_seq_len   0, or a bound every n_b must meet.
 *   row_offsets     device [B+1] one buffer row's offsets (cache_row_offsets /
 *                   buffer_row_offsets[r]), or NULL: the call then reads
 *                   positions [0, p_b + n_b) of every sequence (needs valid_length).
 *   row_positions   device [B] that row's first cache positions
 *                   (cache_offsets[r]), or NULL (0).
 *   row_capacity    0, or a bound row_offsets[B] must meet (buffer_token_size,
 *                   or the rows of K_nope / V).
 *   violations      device int32, ORed with:
 *     MLA_VIOLATION_Q_OFFSETS    valid_length[0] != 0, a decreasing step,
 *                                valid_length[B] != total_q_tokens, or n_b > q_max_seq_len;
 *     MLA_VIOLATION_ROW_OFFSETS  a decreasing step of row_offsets, or
 *                                row_offsets[B] > row_capacity;
 *     MLA_VIOLATION_POSITIONS    a row's positions reach past p_b + n_b (with
 *                                valid_length) or past max_pages_per_seq * page_size;
 *     MLA_VIOLATION_PAGE_IDS     a page id behind a position the call reads is
 *                                >= num_pages.
 *                   The caller zeroes it; the call never clears bits.
 * Enqueues one small kernel (one wave per sequence); no synchronisation, no
 * allocation.  Errors: NULL_ARG, BAD_SHAPE (batch_size > MLA_MAX_BATCH, a
 * zero page size / page count with a page table), HIP.
 */
#define MLA_VIOLATION_Q_OFFSETS 1
#define MLA_VIOLATION_ROW_OFFSETS 2
#define MLA_VIOLATION_POSITIONS 4
#define MLA_VIOLATION_PAGE_IDS 8
mla_status_t mla_prefill_check(const mla_paged_cache_t* kv, const uint32_t* valid_length, uint32_t batch_size,
                               uint32_t total_q_tokens, uint32_t q_max_seq_len, const uint32_t* row_offsets,
                               const uint32_t* row_positions, uint32_t row_capacity, int32_t* violations,
                               void* stream);

/* Debug mode on (nonzero) or off, for every thread of the process; returns the
 * previous setting.  In debug mode each plan, gather, attention and
 * decompression call first runs mla_prefill_check on its own arguments (with
 * the capacity, q_max_seq_len and token count it was given), waits for it
 * (hipStreamSynchronize on the call's stream, so a call in debug mode cannot
 * be captured into a graph), and returns MLA_ERR_PRECONDITION without
 * launching anything when a bit is set.  Debug mode keeps one 4-byte device
 * flag per GPU, allocated on its first use there.  It starts on when the
 * environment variable MLA_PREFILL_DEBUG is "1" as the library loads. */
int mla_prefill_set_debug(int on);

/* Static, human-readable name of a status code (never NULL). */
const char* mla_status_string(mla_status_t status);

/* The HIP error code (hipError_t as int) behind the last MLA_ERR_HIP returned on
 * the calling thread, 0 if none.  For tests of that path: when the environment
 * variable MLA_PREFILL_FAIL_LAUNCH holds a nonzero HIP error code as the library
 * loads, every call that passes its host-side checks returns MLA_ERR_HIP with
 * that code instead of enqueueing anything (no GPU is touched). */
int mla_prefill_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PREFILL_H */
