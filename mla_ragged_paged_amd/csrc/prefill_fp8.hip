// Ragged MLA prefill (causal or null mask) over a paged K_rope cache --
// float8_e4m3fn inputs with per-tensor fp32 scales, bf16 or fp32 output, fp32
// accumulation, optional log-sum-exp output and merge with an earlier partial.
// Semantics: page "flare_mla_prefill" (description; Parameters: q may be
// float8_e4m3fn and the output is then bfloat16; the k_rope_scales overload);
// every fp8 operand stands for code * scale of its tensor.
//
// Same work decomposition and LDS staging as the bf16 kernel (BM = 128 queries
// per workgroup of four waves, BN = 64 keys per tile, two direct-to-LDS stages,
// S^T with one query per lane column) and an online softmax in the exp2 domain;
// what differs:
//   * every weight stays at most 2^RESCALE_LOG2 (below the e4m3 maximum of
//     448): a tile that straddles the diagonal or the end of the keys moves the
//     running reference when its max exceeds it by more than RESCALE_LOG2, and a
//     fully visible tile keeps its weights against the reference as it stands
//     when every lane's sum of them is at most 2^RESCALE_LOG2, else moves the
//     reference up to the tile max and takes them again;
//   * S^T = K . Q^T runs on the fp8 32x32x64 MFMA: two k-steps over the 128
//     nope columns, then one over the 64 rope columns.  The nope partial sum is
//     multiplied by s_knope / s_krope before the rope step, and
//     s_q * s_krope * |scale| * log2(e) is folded into the exp2 argument.
//   * P.V runs on the same fp8 MFMA: p (at most 2^RESCALE_LOG2) is rounded to
//     e4m3 and the row sum is taken over the rounded values, so the weights stay
//     exactly normalised.  A tile that straddles the causal diagonal or the end
//     of the keys while some row of the wave sees fewer than PV8_MIN_KEYS keys
//     -- where the few weights of such a row would be coarse -- uses the bf16
//     MFMA instead, with V converted exactly from e4m3 to bf16 and bf16 p.
//   * V is read transposed with ds_read_b64_tr_b8 (8 keys of one dv column per
//     lane); s_v is applied to O in the epilogue.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int BM = 128;            // queries per workgroup
constexpr int BN = 64;             // keys per tile
constexpr int NT = 256;            // threads per workgroup
constexpr int DQK = 192, DNOPE = 128, DV = 128;
constexpr float RESCALE_LOG2 = 8.0f;
constexpr int32_t PV8_MIN_KEYS = 128;
constexpr float WSUM_MAX = 256.0f;   // 2^RESCALE_LOG2: bound on a lane's e4m3 weight sum over a tile

// LDS stage layout (bytes): rows of fp8, 16-byte chunks XOR-swizzled per row
constexpr int KN_OFF = 0;                      // K_nope [64 rows][8 chunks]
constexpr int KR_OFF = KN_OFF + BN * 128;      // K_rope [64 rows][4 chunks]
// V [64 rows][8 chunks] follows K_rope: at KR_OFF + 64 * 64 (20 KiB stages) when
// K_rope is e4m3, at KR_OFF + 64 * 128 (24 KiB) when it is bf16 (the kernel's QM)

__device__ __forceinline__ int swz_kn(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_kr(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz_krb(int r) { return (r >> 1) & 7; }   // bf16 K_rope rows (8 chunks)
__device__ __forceinline__ int swz_v(int r) { return 2 * (((r >> 1) & 1) | ((r >> 2) & 2)); }

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3 (format code 0 for both operands), unit block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ i32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void bload_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, MLA_LDS void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
}

// four e4m3 bytes -> four bf16 (exact)
__device__ __forceinline__ i32x2 e4m3x4_to_bf16x4(int x) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
  return i32x2{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
}

}  // namespace

// CAUSAL: causal mask, else the null mask.  PLAIN: bf16 output only (no
// log-sum-exp, no earlier partial to merge).  QM: how the query and K_rope come:
//   0  q [T][H][192] e4m3 with q_scale; K_rope e4m3 from the paged cache or
//      from contiguous rows laid out like K (with their scale in k_rope_scale);
//   1  split: q_nope [T][H][128] e4m3 with q_scale and q_rope [T][H][64] bf16;
//      K_rope e4m3 (paged cache or contiguous rows), converted exactly to bf16
//      for the rope product, which runs on the bf16 MFMA;
//   2  split as 1, K_rope bf16 (paged bf16 cache or contiguous rows laid out like K).
// KVSPLIT: the grid holds two units per query tile, and a tile that
// kv_split_tile selects is computed as two halves of its key tiles into the
// workspace (QM 0 only).
template <bool CAUSAL, bool PLAIN, int QM, bool KVSPLIT>
__global__ void __launch_bounds__(NT, 2) prefill_fp8_kernel(PrefillArgs a) {
  // K_rope rows of a stage: 64 bytes (e4m3) or 128 bytes (bf16)
  constexpr int KR_ROW = QM == 2 ? 128 : 64;
  constexpr int V_OFF = KR_OFF + BN * KR_ROW;
  constexpr int STAGE = V_OFF + BN * 128;
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[STAGE];

  // ---- work unit (XCD- and shader-engine-aware order, longest tiles first).
  // Key split: virtual tile 2qt + 1 (launched first) takes tile qt's first half,
  // or the whole tile when it is not split; 2qt takes the second half.
  const uint32_t bid = blockIdx.x;
  WorkUnit u;
  if (!decode_unit(bid, a.heads, a.batch, KVSPLIT ? 2u * a.qtiles : a.qtiles, u)) return;
  const uint32_t h = u.h, b = u.b, qt = KVSPLIT ? u.qt >> 1 : u.qt;
  const uint32_t t0 = a.valid_length[b];
  const uint32_t n = a.valid_length[b + 1] - t0;
  const uint32_t i0 = qt * BM;
  if (i0 >= n) return;

  const uint32_t H = a.heads;
  const int32_t p = (int32_t)a.cache_lengths[b];
  const uint32_t g0 = a.cache_row_offsets[b];
  const int32_t len = (int32_t)(a.cache_row_offsets[b + 1] - g0);
  const int32_t c0 = a.cache_offsets ? (int32_t)a.cache_offsets[b] : 0;
  // row mode: a row holding none of the sequence's keys leaves its outputs alone;
  // row_first: this row's slice starts at cache position 0 (no earlier partial)
  bool row_first = true;
  if constexpr (!PLAIN) {
    if (a.row_mode) {
      if (len == 0) return;
      row_first = c0 == 0;
    }
  }
  const int32_t i_last = (int32_t)min(n, i0 + BM) - 1;
  // causal: the keys some query of the tile can see, c0 + j <= p + i_last;
  // null mask: every key the row holds for the sequence
  constexpr bool causal = CAUSAL;
  const int32_t jend = causal ? max(0, min(p + i_last - c0 + 1, len)) : len;
  const int32_t nkt = (jend + BN - 1) / BN;
  int32_t kt_lo = 0, kt_hi = nkt;                     // this unit's key tiles
  bool part = false;                                  // key split: writes a partial
  if constexpr (KVSPLIT) {
    part = kv_split_tile(jend, a.split_keys);
    const int32_t mid = (nkt + 1) >> 1;
    if (part) {
      kt_lo = (u.qt & 1u) ? 0 : mid;
      kt_hi = (u.qt & 1u) ? mid : nkt;
    } else if ((u.qt & 1u) == 0) {
      return;
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, hf = lane >> 5;
  const int32_t iw0 = (int32_t)i0 + 32 * w;
  const bool wave_rows = iw0 < (int32_t)n;
  const int32_t my_i = iw0 + li;
  const int32_t wq_first = p + iw0;
  const int32_t wq_last = p + min((int32_t)n, iw0 + 32) - 1;

  // per-tensor dequantisation scales (a bf16 K_rope carries none)
  const float s_q = *a.q_scale, s_kn = *a.k_nope_scale, s_v = *a.v_scale;
  const float s_kr = QM == 2 ? 1.f : *a.k_rope_scale;

  constexpr uint32_t QW = QM == 0 ? DQK : DNOPE;      // e4m3 columns of one row of the tensor at a.q
  const uint32_t q_row = H * QW, kv_row = H * DNOPE;
  const auto q_rs = rsrc(static_cast<const uint8_t*>(a.q) + ((size_t)t0 * H + h) * QW, (n - 1) * q_row + QW);
  const uint32_t qr_row = H * (DQK - DNOPE) * 2;       // bf16 q_rope (split query)
  const auto qr_rs = rsrc(QM != 0 ? static_cast<const uint8_t*>(a.q_rope) + ((size_t)t0 * H + h) * (DQK - DNOPE) * 2
                                  : nullptr,
                          QM != 0 ? (n - 1) * qr_row + (DQK - DNOPE) * 2 : 0u);
  // contiguous K_rope rows (e4m3, or bf16 with QM 2): key j of the sequence is row g0 + j
  const bool contig = a.rope_rows != nullptr;
  // bytes of the unit's K_nope / V rows from its first key (64-bit: one sequence's
  // keys in a buffer row may span more than 4 GiB at 128 heads)
  const uint64_t kv_bytes = jend > 0 ? (uint64_t)(jend - 1) * kv_row + DNOPE : 0u;
  const uint8_t* kn_base = static_cast<const uint8_t*>(a.k_nope) + ((size_t)g0 * H + h) * DNOPE;
  const uint8_t* v_base = static_cast<const uint8_t*>(a.v) + ((size_t)g0 * H + h) * DNOPE;
  // paged K_rope: one descriptor over the cache layer; contiguous rows: one per
  // tile, starting at the tile's first row (built in issue_rope, so the 32-bit
  // byte count never has to cover more than what remains of the sequence's rows)
  const auto cr_rs = rsrc(a.cache, a.cache_bytes);
  const uint8_t* rr_base = contig ? static_cast<const uint8_t*>(a.rope_rows) + (size_t)g0 * KR_ROW : nullptr;
  const uint32_t* __restrict__ PT = a.page_table + (size_t)b * a.max_pages;
  const uint32_t cache_row = a.row_width * (QM == 2 ? 2u : 1u);   // bytes of one cache row

  // ---- Q^T operands: lane (li, hf) holds bytes [64ks + 32hf, +32) of its query.
  // Loaded after the first tile's page ids and K_nope / V loads (vector-memory
  // waits are in issue order); a negative scale's sign is applied once Q is in.
  // Split query: qop[0..1] hold q_nope's bytes as above, and qr[r] holds q_rope
  // columns [16r + 8hf, +8) in bf16 (the 32x32x16 bf16 MFMA's B operand).
  constexpr int QKS = QM == 0 ? 3 : 2;                // e4m3 k-steps held in qop
  i32x8 qop[3];
  bf16x8 qr[4];
  auto load_q = [&]() {
    const uint32_t qoff = (uint32_t)my_i * q_row + hf * 32;
#pragma unroll
    for (int ks = 0; ks < QKS; ++ks) {
      const i32x4 x0 = bload16(q_rs, qoff + ks * 64);
      const i32x4 x1 = bload16(q_rs, qoff + ks * 64 + 16);
      qop[ks] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
    if constexpr (QM != 0) {
      const uint32_t qroff = (uint32_t)my_i * qr_row + hf * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) qr[r] = __builtin_bit_cast(bf16x8, bload16(qr_rs, qroff + r * 32));
    }
  };

  // ---- this lane's slots of a tile load (one 1 KiB load = 64 slots of 16 B)
  uint32_t kn_off[2], v_off[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {                      // K_nope / V load m = 2w + u: rows 8m .. 8m+7
    const int r = 16 * w + 8 * u + (lane >> 3);
    const int cs = lane & 7;
    kn_off[u] = (uint32_t)r * kv_row + 16u * (uint32_t)(cs ^ swz_kn(r));
    v_off[u] = (uint32_t)r * kv_row + 16u * (uint32_t)(cs ^ swz_v(r));
  }
  // K_rope, e4m3 rows: load m = w covers rows 16m .. 16m+15, slot lane -> row
  // 16m + lane/4.  bf16 rows (QM 2): loads m = 2w + u cover rows 8m .. 8m+7, slot
  // lane -> row 8m + lane/8, chunk (lane % 8) ^ swz_krb(row).
  constexpr int KRL = QM == 2 ? 2 : 1;               // K_rope loads per wave and tile
  int kr_row[KRL], kr_chunk[KRL];
#pragma unroll
  for (int u = 0; u < KRL; ++u) {
    if constexpr (QM == 2) {
      kr_row[u] = 16 * w + 8 * u + (lane >> 3);
      kr_chunk[u] = (lane & 7) ^ swz_krb(kr_row[u]);
    } else {
      kr_row[u] = 16 * w + (lane >> 2);
      kr_chunk[u] = (lane & 3) ^ swz_kr(kr_row[u]);
    }
  }
  auto page_of = [&](int32_t kt, int u) -> uint32_t {
    if (contig) return 0u;
    const int32_t j = min(kt * BN + kr_row[u], jend - 1);
    const uint32_t pos = (uint32_t)(c0 + j);
    return a.page_shift < 32u ? PT[pos >> a.page_shift] : PT[pos / a.page_size];
  };
  // K_nope and V rows of tile kt, then its K_rope rows (which need the page id).
  // Rows past the keys are filled with zeros by the range-checked loads, so no
  // stage ever holds stale or uninitialised V rows.
  // The tile's descriptors start at its first row (scalar arithmetic; the byte
  // count shrinks with it, so the range check still ends at the last key -- and
  // is capped at 4 GiB - 1 while more remains, far beyond the few MiB a tile
  // reads past its first row), and the LDS destinations come from the
  // wave-uniform index.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto issue_kv = [&](int32_t kt, uint8_t* stage) {
    const uint64_t jrow = (uint64_t)(kt * BN) * kv_row;   // < kv_bytes for every tile of the unit
    const uint32_t left = (uint32_t)min(kv_bytes - jrow, (uint64_t)0xFFFFFFFFu);
    const auto kn_t = rsrc(kn_base + jrow, left);
    const auto v_t = rsrc(v_base + jrow, left);
    MLA_LDS uint8_t* st = (MLA_LDS uint8_t*)stage;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int m = 2 * wu + u;
      bload_lds(kn_t, kn_off[u], st + KN_OFF + m * 1024);
      bload_lds(v_t, v_off[u], st + V_OFF + m * 1024);
    }
  };
  auto issue_rope = [&](int32_t kt, uint8_t* stage, const uint32_t (&pg)[2]) {
    MLA_LDS uint8_t* st = (MLA_LDS uint8_t*)stage;
    const auto kr_t = contig ? rsrc(rr_base + (size_t)(kt * BN) * KR_ROW,
                                    (uint32_t)min((uint64_t)(jend - kt * BN) * KR_ROW, (uint64_t)0xFFFFFFFFu))
                             : cr_rs;
#pragma unroll
    for (int u = 0; u < KRL; ++u) {
      uint32_t off;
      if (contig) {
        // the tile's descriptor ends at the last key: rows past it read as zeros
        off = (uint32_t)kr_row[u] * (uint32_t)KR_ROW + 16u * kr_chunk[u];
      } else {
        const int32_t j = min(kt * BN + kr_row[u], jend - 1);
        const uint32_t pos = (uint32_t)(c0 + j);
        const uint32_t slot = a.page_shift < 32u ? (pos & (a.page_size - 1u)) : (pos % a.page_size);
        const uint32_t el = QM == 2 ? 2u : 1u;
        off = (pg[u] * a.page_size + slot) * cache_row + a.rope_col * el + 16u * kr_chunk[u];
      }
      bload_lds(kr_t, off, st + KR_OFF + (KRL * wu + u) * 1024);
    }
  };

  // ---- LDS read offsets.  K operand (fp8 32x32x64): row R = 32kb + li, bytes
  // [64ks + 32hf, +32) = chunks 4ks + 2hf and +1 (nope), 2hf and +1 (rope).
  uint32_t kn_rd[2][2], kr_rd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int x = 0; x < 2; ++x) kn_rd[ks][x] = KN_OFF + li * 128 + 16 * ((4 * ks + 2 * hf + x) ^ swz_kn(li));
#pragma unroll
  for (int x = 0; x < 2; ++x) kr_rd[x] = KR_OFF + li * 64 + 16 * ((2 * hf + x) ^ swz_kr(li));
  // split query, bf16 rope product (32x32x16): K operand row R = 32kb + li,
  // columns [16r + 8hf, +8): e4m3 rows (QM 1) give 8 bytes at chunk r ^ swz_kr(R),
  // half hf; bf16 rows (QM 2) 16 bytes at chunk (2r + hf) ^ swz_krb(R)
  uint32_t krs_rd[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    krs_rd[r] = QM == 2 ? KR_OFF + li * 128 + 16 * ((2 * r + hf) ^ swz_krb(li))
                        : KR_OFF + li * 64 + 16 * (r ^ swz_kr(li)) + 8 * hf;
  // V transposed byte reads (ds_read_b64_tr_b8: lane 16g + 2e + c supplies row e,
  // bytes 8c..8c+7; lane 16g + i receives column i of the 8 rows).  For 16-key
  // step t: rows 16t + 4(g>>1) + (e&3) + 8(e>>2), dv = 32d + 16(g&1) + 8c.
  const int tr_g = lane >> 4, tr_e = (lane >> 1) & 7, tr_c = lane & 1;
  const int tr_row = 4 * (tr_g >> 1) + (tr_e & 3) + 8 * (tr_e >> 2);
  // swz_v(r + 16t) == swz_v(r), so v_rd[d] + t * 16 * 128 addresses step t.
  uint32_t v_rd[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int chunk = 2 * d + (tr_g & 1);
    v_rd[d] = V_OFF + tr_row * 128 + 16 * (chunk ^ swz_v(tr_row)) + 8 * tr_c;
  }

  // ---- softmax state
  // exp2 factor for the combined score, and the factor taking the nope partial
  // sum to the units of the rope one (q_scale applies to both halves of a full
  // query, to q_nope only in a split one)
  const float c = QM == 0 ? a.scale_log2 * s_q * s_kr : a.scale_log2 * s_kr;
  const float ratio = QM == 0 ? s_kn / s_kr : s_q * s_kn / s_kr;
  const float thr = RESCALE_LOG2 / c;
  float m_run = -1e30f, mc = m_run * c, l_run = 0.f;
  bool fresh = true;                                 // no tile computed yet
  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x16{};
  // Row sums of the e4m3 weights of fully visible tiles, taken on the matrix core:
  // (all-ones 32 x 64) . P^T puts each query column's sum over the tile's 64 keys
  // in every row of the column, so lane (li, hf) reads its query's sum in
  // lsum[0] (only that element is rescaled and read; both halves hold the whole
  // sum).  Under the causal mask the register budget has room for the extra
  // accumulator and operand; the null-mask kernels sum on the VALU.
  constexpr bool MFMA_ROWSUM = CAUSAL;
  f32x16 lsum = f32x16{};
  const int one4 = 0x38383838;                       // four e4m3 1.0
  i32x8 ones8 = {one4, one4, one4, one4, one4, one4, one4, one4};

  // ---- prologue, ordered for the first tile's critical path: page ids first,
  // then the K_nope / V rows, then Q, so the K_rope loads wait for the page ids only
  uint32_t pg_next[2] = {0u, 0u};
  if (kt_hi > kt_lo) {
    uint32_t pg0[2] = {0u, 0u};
#pragma unroll
    for (int u = 0; u < KRL; ++u) {
      pg0[u] = page_of(kt_lo, u);
      pg_next[u] = page_of(kt_lo + 1, u);
    }
    // all four waves start their first tile together
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    issue_kv(kt_lo, stage0);
    __builtin_amdgcn_sched_barrier(0);
    load_q();
    __builtin_amdgcn_sched_barrier(0);
    issue_rope(kt_lo, stage0, pg0);
  }
  // with no key to attend to, Q is never read (the epilogue writes 0, or passes
  // an earlier partial through)

  auto step = [&](int32_t kt, const uint8_t* st, uint8_t* next) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the all-ones operand stays in its registers across tiles instead of being
    // rebuilt with eight moves in each
    if constexpr (MFMA_ROWSUM) asm volatile("" : "+v"(ones8));
    if (kt == kt_lo && a.scale < 0.f) {
#pragma unroll
      for (int ks = 0; ks < QKS; ++ks) qop[ks] ^= (int)0x80808080;
      if constexpr (QM != 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          qr[r] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(i32x4, qr[r]) ^ (int)0x80008000);
      }
    }
    if (kt + 1 < kt_hi) {
      issue_kv(kt + 1, next);
      issue_rope(kt + 1, next, pg_next);
#pragma unroll
      for (int u = 0; u < KRL; ++u) pg_next[u] = page_of(kt + 2, u);
    }
    const int32_t j0 = kt * BN;
    if (!(wave_rows && (!causal || c0 + j0 <= wq_last))) return;
    // S^T: two nope k-steps, scale to rope units, the rope k-step(s)
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < QKS; ++ks) {
      i32x8 kf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t o0 = ks < 2 ? kn_rd[ks][0] + kb * 32 * 128 : kr_rd[0] + kb * 32 * 64;
        const uint32_t o1 = ks < 2 ? kn_rd[ks][1] + kb * 32 * 128 : kr_rd[1] + kb * 32 * 64;
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(st + o0);
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(st + o1);
        kf[kb] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
      if (ks == 2) {
        s[0] *= ratio;
        s[1] *= ratio;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_fp8(kf[kb], qop[ks], s[kb]);
    }
    if constexpr (QM != 0) {
      // split query: nope sum to rope units, then four bf16 k-steps over the rope
      // columns (e4m3 K_rope converted exactly to bf16 on the way)
      s[0] *= ratio;
      s[1] *= ratio;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 kfr;
          if constexpr (QM == 2) {
            kfr = *reinterpret_cast<const bf16x8*>(st + krs_rd[r] + kb * 32 * 128);
          } else {
            const i32x2 x = *reinterpret_cast<const i32x2*>(st + krs_rd[r] + kb * 32 * 64);
            const i32x2 lo = e4m3x4_to_bf16x4(x[0]), hi = e4m3x4_to_bf16x4(x[1]);
            kfr = __builtin_bit_cast(bf16x8, i32x4{lo[0], lo[1], hi[0], hi[1]});
          }
          s[kb] = mfma_bf16(kfr, qr[r], s[kb]);
        }
      }
    }
    const bool full = (j0 + BN <= len) && (!causal || c0 + j0 + BN - 1 <= wq_first);
    // e4m3 weights and P.V also on a straddling tile when every row of the wave
    // sees at least PV8_MIN_KEYS keys in this call (its first row sees the
    // fewest): its weights are then as coarse as those of any fully visible tile
    const bool pv8 = full || min(causal ? p + iw0 - c0 + 1 : len, len) >= PV8_MIN_KEYS;
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int32_t kbase = j0 + 32 * kb + 4 * hf;
        const int32_t lim = causal ? min(len - 1 - kbase, p + my_i - c0 - kbase) : len - 1 - kbase;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t roff = 8 * (r >> 2) + (r & 3);
          s[kb][r] = roff <= lim ? s[kb][r] : -INFINITY;
        }
      }
    }
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float e[2][16];
    auto weights = [&]() {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) e[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
    };
    // fp8 P: byte 16kb + r of this lane is key 32kb + 8(r/4) + 4hf + r%4; each
    // word's four weights are packed as soon as they are taken, so the scores
    // (kept for a second pass) and few weights are live at once
    int pq[8];
    float ps = 0.f;                                   // VALU row sum (this lane's 32 keys)
    auto weights_fp8 = [&]() {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int kb = x >> 2, r = 4 * (x & 3);
        float w4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w4[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + k], c, -mc));
        // the first conversion's untouched half is overwritten by the second, so
        // its "old" operand is any dead register (no copy of a zero needed)
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(w4[0], w4[1], __builtin_bit_cast(int, w4[0]), false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(w4[2], w4[3], wd, true);
        pq[x] = wd;
      }
      if constexpr (MFMA_ROWSUM) {
        lsum = mfma_fp8(ones8, i32x8{pq[0], pq[1], pq[2], pq[3], pq[4], pq[5], pq[6], pq[7]}, lsum);
      } else {
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pq[x], 1.0f, false), ones, ps0, false);
          ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pq[x], 1.0f, true), ones, ps1, false);
        }
        ps = ps0 + ps1;
      }
    };
    // A fully visible tile first takes its e4m3 weights against the running
    // reference as it stands; when every lane's sum of them is at most
    // 2^RESCALE_LOG2 (so no weight exceeds it: an overflowing conversion gives a
    // NaN or 448, which fails the test too) they stand, and the tile needs no
    // max.  Otherwise -- and on the wave's first tile, and on every tile that
    // straddles the diagonal or the end of the keys -- the tile max is taken:
    // a fully visible tile moves the reference up to it, a straddling one when
    // it exceeds the reference by more than RESCALE_LOG2, and the weights are
    // taken again.
    bool redo = !full || fresh;
    fresh = false;
    float prev = 0.f;
    if (!redo) {
      if constexpr (MFMA_ROWSUM) prev = lsum[0];
      weights_fp8();
      const float d = MFMA_ROWSUM ? lsum[0] - prev : ps;
      redo = __builtin_amdgcn_ballot_w64(!(d <= WSUM_MAX)) != 0;
      if constexpr (MFMA_ROWSUM) {
        if (redo) lsum[0] = prev;
      }
    }
    if (redo) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_across_halves(mx);
      if (__builtin_amdgcn_ballot_w64(mx > (full ? m_run : m_run + thr)) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        m_run = m_new;
        mc = m_run * c;
        l_run *= alpha;
        if constexpr (MFMA_ROWSUM) lsum[0] *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] *= alpha;
      }
      if (pv8)
        weights_fp8();
      else
        weights();
    }

    if (pv8) {
      const i32x8 pop = {pq[0], pq[1], pq[2], pq[3], pq[4], pq[5], pq[6], pq[7]};
      if constexpr (!MFMA_ROWSUM) l_run += ps;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        int va[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (MLA_LDS i32x2*)((const MLA_LDS uint8_t*)st + v_rd[d] + t * 16 * 128));
          va[2 * t] = v2[0];
          va[2 * t + 1] = v2[1];
        }
        o[d] = mfma_fp8(i32x8{va[0], va[1], va[2], va[3], va[4], va[5], va[6], va[7]}, pop, o[d]);
      }
    } else {
      // bf16 P with V converted exactly from e4m3
      uint32_t pw[16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 8; ++x) pw[8 * kb + x] = pack_bf16x2(e[kb][2 * x], e[kb][2 * x + 1]);
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int x = 0; x < 16; x += 2) {
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[x]), ones, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[x + 1]), ones, ps1, false);
      }
      l_run += ps0 + ps1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const i32x4 pv = {(int)pw[4 * t], (int)pw[4 * t + 1], (int)pw[4 * t + 2], (int)pw[4 * t + 3]};
        const bf16x8 pop = __builtin_bit_cast(bf16x8, pv);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (MLA_LDS i32x2*)((const MLA_LDS uint8_t*)st + v_rd[d] + t * 16 * 128));
          const i32x2 lo = e4m3x4_to_bf16x4(v2[0]), hi = e4m3x4_to_bf16x4(v2[1]);
          const bf16x8 va = __builtin_bit_cast(bf16x8, i32x4{lo[0], lo[1], hi[0], hi[1]});
          o[d] = mfma_bf16(va, pop, o[d]);
        }
      }
    }
  };
  for (int32_t kt = kt_lo; kt < kt_hi; kt += 2) {
    step(kt, stage0, stage1);
    if (kt + 1 < kt_hi) step(kt + 1, stage1, stage0);
  }

  // ---- epilogue: row sums of both halves, normalise (applying s_v), store the
  // row with its log-sum-exp (merged with an earlier partial when one is given)
  const float l_tot = l_run + swap_halves(l_run) + (MFMA_ROWSUM ? lsum[0] : 0.f);
  if constexpr (PLAIN && !KVSPLIT) {
    // Plain bf16 rows go through LDS (the stages are free once every wave is past
    // its last tile): waves 0-1 (tile rows 0..63) in stage 0, waves 2-3 in stage
    // 1, row r at (r % 64) * 256 with 16-byte chunk c at c ^ (r % 16).  Then 16
    // lanes store each query's whole 256-byte row with streaming stores, which
    // keep the output out of L2 (measured 1.5 % faster than plain stores from
    // the registers).
    const float inv = l_tot > 0.f ? s_v / l_tot : 0.f;
    __syncthreads();
    const int row = 32 * w + li;
    MLA_LDS uint8_t* ot = (MLA_LDS uint8_t*)(row < 64 ? stage0 : stage1);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t w0 = pack_bf16x2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv);
        *reinterpret_cast<MLA_LDS u32x2*>(ot + (row & 63) * 256 + 16 * ((4 * d + g) ^ (row & 15)) + 8 * hf) =
            u32x2{w0, w1};
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = 16 * it + (tid >> 4), cc = tid & 15;
      const MLA_LDS uint8_t* src = (const MLA_LDS uint8_t*)(r < 64 ? stage0 : stage1);
      if ((int32_t)i0 + r < (int32_t)n) {
        const i32x4 v = *reinterpret_cast<const MLA_LDS i32x4*>(src + (r & 63) * 256 + 16 * (cc ^ (r & 15)));
        __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(static_cast<uint16_t*>(a.out) +
                                                                 ((size_t)(t0 + i0 + r) * H + h) * 128 + 8 * cc));
      }
    }
    return;
  }
  // Row mode, per query: the row holding the query's last visible key (p + i under
  // the causal mask, the context's last under the null mask) finishes it and
  // writes the output; earlier rows carry its partial, and later rows -- which
  // hold none of its keys -- leave it alone.
  bool row_last = true, row_skip = false;
  if constexpr (!PLAIN) {
    if (a.row_mode) {
      const int32_t k_last = causal ? p + my_i : p + (int32_t)n - 1;
      row_skip = k_last < c0;
      row_last = k_last < c0 + len;
    }
  }
  if (my_i < (int32_t)n && !row_skip) {
    const float inv = l_tot > 0.f ? s_v / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? mc + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    if (KVSPLIT && part)
      store_output_row<false>(kv_split_target(a, (u.qt & 1u) ^ 1u), (size_t)(t0 + my_i) * H + h, hf, o, inv, lse2);
    else
      store_output_row<PLAIN>(row_target(a, row_first, row_last), (size_t)(t0 + my_i) * H + h, hf, o, inv, lse2);
  }
}

hipError_t launch_prefill_fp8(PrefillArgs a, uint32_t q_max, hipStream_t stream) {
  a.qtiles = (q_max + BM - 1) / BM;
  const bool kv_split = a.split_keys != 0;
  const uint64_t units = (uint64_t)a.heads * a.batch * a.qtiles * (kv_split ? 2u : 1u);
  const uint64_t grid = (units + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  const bool plain = !a.out_fp32 && !a.lse && !a.prev_out && !a.row_mode;
  if (kv_split) {
    // full query, no row mode, no earlier partial (the entry point checks)
    auto kernel = a.causal ? (plain ? prefill_fp8_kernel<true, true, 0, true> : prefill_fp8_kernel<true, false, 0, true>)
                           : (plain ? prefill_fp8_kernel<false, true, 0, true> : prefill_fp8_kernel<false, false, 0, true>);
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(NT), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_kv_split_merge(a, stream);
  }
  auto pick = [&](auto qm) {
    constexpr int QM = decltype(qm)::value;
    return a.causal ? (plain ? prefill_fp8_kernel<true, true, QM, false> : prefill_fp8_kernel<true, false, QM, false>)
                    : (plain ? prefill_fp8_kernel<false, true, QM, false> : prefill_fp8_kernel<false, false, QM, false>);
  };
  auto kernel = a.q_split == 0 ? pick(std::integral_constant<int, 0>{})
                               : a.q_split == 1 ? pick(std::integral_constant<int, 1>{})
                                                : pick(std::integral_constant<int, 2>{});
  hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
