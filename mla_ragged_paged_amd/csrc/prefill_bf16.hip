// Ragged MLA prefill over a paged K_rope cache -- bf16 inputs, bf16 or fp32
// output, fp32 accumulation.  Semantics: page "flare_mla_prefill" (description
// and Args) with the paged k_rope operand; argument meanings of page
// "mla_prefill_v2_ragged" (Args), whose mask predicate is causal or null here.
// Each query row's log-sum-exp can be written too, and the row merged with an
// earlier partial result (another buffer row's keys) in the epilogue.
//
// Work unit = (head h, sequence b, query tile of BM = 128 rows).  A workgroup of
// four waves owns one unit; wave w owns queries [32w, 32w+32) of the tile.
//
// Keys stream through LDS in tiles of BN = 64, two stages deep.  Each tile is
// three regions -- K_nope [64][128], K_rope [64][64] (read through the page
// table, shared by all heads) and V [64][128] -- filled by buffer loads that
// write LDS directly (no register staging).  A 16-byte chunk c of row r is
// stored at chunk c ^ swz(r) of its row, which keeps both the MFMA operand reads
// and the transposed V reads free of bank conflicts without padding.  One
// barrier per tile: it publishes tile k and retires tile k-1's stage, which the
// loads of tile k+1 then overwrite while tile k is consumed.
//
// Per wave and key tile, on the 32x32x16 bf16 MFMA:
//   S^T = K . Q^T  (A = K rows from LDS, B = the wave's Q held in registers),
//        so each lane owns one query column and 32 of the tile's 64 keys:
//        row max / sum need one exchange between the wave's two 32-lane halves;
//   online softmax in the exp2 domain: p = exp2(s*c - m*c), c = |scale|*log2(e)
//        (a negative scale is applied by flipping the sign of Q, which is
//        exact).  The reference m is set to the row max on the first tile
//        and moves only when the weights some lane computes for a tile sum
//        to more than 2^16 (or are not finite): then m becomes the running
//        max, O and the row sum are rescaled and the tile's weights are
//        computed again.  Most tiles take neither the max nor the rescale.
//        p is rounded to bf16 once and the row sum is taken over the rounded
//        values (v_dot2 against (1, 1)), so the weights applied to V are
//        normalised exactly.  Masks are applied only on tiles that straddle
//        the causal diagonal or the end of the sequence's keys (under the
//        null mask only the end of the keys);
//   O^T += V^T . P^T (A = V read transposed out of row-major LDS with
//        ds_read_b64_tr_b16, B = P^T straight from the S^T registers).  The 16
//        keys of one MFMA step are taken in the order the S^T accumulator
//        holds them; V is read in that same order.
// Buffer descriptors are sized to the valid rows, so loads past the ragged
// tail return zeros without branches.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int BM = 128;            // queries per workgroup
constexpr int BN = 64;             // keys per tile
constexpr int NT = 256;            // threads per workgroup
constexpr int DQK = 192, DNOPE = 128, DV = 128;
constexpr float WSUM_MAX = 65536.0f;   // 2^16: bound on one lane's weight sum over a tile

// LDS stage layout (bytes)
constexpr int KN_OFF = 0;                      // K_nope [64 rows][16 chunks of 16 B]
constexpr int KR_OFF = KN_OFF + BN * 256;      // K_rope [64 rows][8 chunks]
constexpr int V_OFF = KR_OFF + BN * 128;       // V      [64 rows][16 chunks]
constexpr int STAGE = V_OFF + BN * 256;        // 40 KiB
constexpr int LDS_BYTES = 2 * STAGE;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ i32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 64 lanes x 16 B from the buffer at per-lane byte offsets into 1 KiB of LDS at `dst`
// (lane i lands at dst + 16 i).
__device__ __forceinline__ void bload_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, MLA_LDS void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
}

}  // namespace

// CAUSAL: causal mask, else the null mask.  PLAIN: bf16 output only (no
// log-sum-exp, no earlier partial to merge).  QSPLIT: the query comes as q_nope
// [T][H][128] and q_rope [T][H][64].  K_rope is read through the page table, or
// from contiguous rows laid out like K when a.rope_rows is set.  KVSPLIT: the grid
// holds two units per query tile, and a tile that kv_split_tile selects is
// computed as two halves of its key tiles into the workspace (full query only).
template <bool CAUSAL, bool PLAIN, bool QSPLIT, bool KVSPLIT>
__global__ void __launch_bounds__(NT, 2) prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

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
  const int32_t iw0 = (int32_t)i0 + 32 * w;          // wave's first query
  const bool wave_rows = iw0 < (int32_t)n;
  const int32_t my_i = iw0 + li;                      // this lane's query column
  const int32_t wq_first = p + iw0;
  const int32_t wq_last = p + min((int32_t)n, iw0 + 32) - 1;

  // ---- buffer descriptors (byte offsets relative to this unit's first row)
  // (split Q: q_rs covers q_nope rows of 128 columns, qr_rs the q_rope rows)
  constexpr uint32_t QW = QSPLIT ? DNOPE : DQK;       // columns of one row of the tensor at a.q
  const uint32_t q_row = H * QW * 2, kv_row = H * DNOPE * 2;
  const auto q_rs = rsrc(static_cast<const uint8_t*>(a.q) + ((size_t)t0 * H + h) * QW * 2, (n - 1) * q_row + QW * 2);
  const uint32_t qr_row = H * (DQK - DNOPE) * 2;
  const auto qr_rs = rsrc(QSPLIT ? static_cast<const uint8_t*>(a.q_rope) + ((size_t)t0 * H + h) * (DQK - DNOPE) * 2
                                 : nullptr,
                          QSPLIT ? (n - 1) * qr_row + (DQK - DNOPE) * 2 : 0u);
  // contiguous K_rope rows laid out like K: key j of the sequence is row g0 + j, 128 bytes
  const bool contig = a.rope_rows != nullptr;
  // bytes of the unit's K_nope / V rows from its first key (64-bit: one sequence's
  // keys in a buffer row may span more than 4 GiB at 128 heads)
  const uint64_t kv_bytes = jend > 0 ? (uint64_t)(jend - 1) * kv_row + DNOPE * 2 : 0u;
  // paged K_rope: one descriptor over the cache layer; contiguous rows: one per
  // tile, starting at the tile's first row (built in issue_rope, so the 32-bit
  // byte count never has to cover more than what remains of the sequence's rows)
  const auto cr_rs = rsrc(a.cache, a.cache_bytes);
  const uint8_t* rr_base = contig ? static_cast<const uint8_t*>(a.rope_rows) + (size_t)g0 * 128 : nullptr;
  const uint32_t* __restrict__ PT = a.page_table + (size_t)b * a.max_pages;
  const uint32_t cache_row = a.row_width * 2;

  // ---- Q^T operands: lane (li, hf) holds q[t][h][16ks + 8hf .. +7] for its query
  // (rows past the sequence read as zeros).  Loaded after the first tile's
  // page ids and K_nope / V loads (vector-memory waits are in issue order).
  bf16x8 qop[12];
  auto load_q = [&]() {
    const uint32_t qoff = (uint32_t)my_i * q_row + hf * 16;
    if constexpr (QSPLIT) {
      const uint32_t qroff = (uint32_t)my_i * qr_row + hf * 16;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qop[ks] = __builtin_bit_cast(bf16x8, bload16(q_rs, qoff + ks * 32));
#pragma unroll
      for (int ks = 8; ks < 12; ++ks) qop[ks] = __builtin_bit_cast(bf16x8, bload16(qr_rs, qroff + (ks - 8) * 32));
    } else {
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) qop[ks] = __builtin_bit_cast(bf16x8, bload16(q_rs, qoff + ks * 32));
    }
  };

  // ---- this lane's slots of a tile load (one 1 KiB load = 64 slots of 16 B)
  // K_nope / V: load m = 4w + u covers rows 4m .. 4m+3, slot lane -> row 4m + lane/16,
  // stored chunk lane%16 holds source chunk (lane%16) ^ swz(row).
  uint32_t kn_off[4], v_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 16 * w + 4 * u + (lane >> 4);
    const int cs = lane & 15;
    kn_off[u] = (uint32_t)r * kv_row + 16u * (uint32_t)(cs ^ (r & 15));
    v_off[u] = (uint32_t)r * kv_row + 16u * (uint32_t)(cs ^ (4 * (r & 3)));
  }
  // K_rope: load m = 2w + u covers rows 8m .. 8m+7, slot lane -> row 8m + lane/8
  int kr_row[2], kr_chunk[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 16 * w + 8 * u + (lane >> 3);
    kr_row[u] = r;
    kr_chunk[u] = (lane & 7) ^ ((r >> 1) & 7);
  }
  auto page_of = [&](int32_t kt, int u) -> uint32_t {
    if (contig) return 0u;
    const int32_t j = min(kt * BN + kr_row[u], jend - 1);   // clamped: always a valid position
    const uint32_t pos = (uint32_t)(c0 + j);
    return a.page_shift < 32u ? PT[pos >> a.page_shift] : PT[pos / a.page_size];
  };
  // K_nope and V rows of tile kt, then its K_rope rows (which need the page ids).
  // Rows past the keys are filled with zeros by the range-checked loads, so no
  // stage ever holds stale or uninitialised V rows.
  // The tile's descriptors start at its first row (scalar arithmetic; the byte
  // count shrinks with it, so the range check still ends at the last key -- and
  // is capped at 4 GiB - 1 while more remains, far beyond the few MiB a tile
  // reads past its first row), and the LDS destinations come from the
  // wave-uniform index.
  const uint8_t* kn_base = static_cast<const uint8_t*>(a.k_nope) + ((size_t)g0 * H + h) * DNOPE * 2;
  const uint8_t* v_base = static_cast<const uint8_t*>(a.v) + ((size_t)g0 * H + h) * DNOPE * 2;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto issue_kv = [&](int32_t kt, MLA_LDS uint8_t* st) {
    const uint64_t jrow = (uint64_t)(kt * BN) * kv_row;   // < kv_bytes for every tile of the unit
    const uint32_t left = (uint32_t)min(kv_bytes - jrow, (uint64_t)0xFFFFFFFFu);
    const auto kn_t = rsrc(kn_base + jrow, left);
    const auto v_t = rsrc(v_base + jrow, left);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int m = 4 * wu + u;
      bload_lds(kn_t, kn_off[u], st + KN_OFF + m * 1024);
      bload_lds(v_t, v_off[u], st + V_OFF + m * 1024);
    }
  };
  auto issue_rope = [&](int32_t kt, MLA_LDS uint8_t* st, const uint32_t (&pg)[2]) {
    const auto kr_t = contig ? rsrc(rr_base + (size_t)(kt * BN) * 128,
                                    (uint32_t)min((uint64_t)(jend - kt * BN) * 128u, (uint64_t)0xFFFFFFFFu))
                             : cr_rs;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int m = 2 * wu + u;
      uint32_t off;
      if (contig) {
        // the tile's descriptor ends at the last key: rows past it read as zeros
        off = (uint32_t)kr_row[u] * 128u + 16u * kr_chunk[u];
      } else {
        const int32_t j = min(kt * BN + kr_row[u], jend - 1);
        const uint32_t pos = (uint32_t)(c0 + j);
        const uint32_t slot = a.page_shift < 32u ? (pos & (a.page_size - 1u)) : (pos % a.page_size);
        off = (pg[u] * a.page_size + slot) * cache_row + a.rope_col * 2 + 16u * kr_chunk[u];
      }
      bload_lds(kr_t, off, st + KR_OFF + m * 1024);
    }
  };

  // ---- per-lane LDS read offsets (within a stage)
  // K operand: row R = 32kb + li, chunk 2ks + hf stored at chunk ^ swz(R)
  uint32_t kn_rd[8], kr_rd[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kn_rd[ks] = KN_OFF + li * 256 + 16 * ((2 * ks + hf) ^ (li & 15));
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kr_rd[ks] = KR_OFF + li * 128 + 16 * ((2 * ks + hf) ^ ((li >> 1) & 7));
  // V transposed reads (ds_read_b64_tr_b16: lane 16g+4e+c of a 16-lane group supplies
  // row e, columns 4c..4c+3): row = 16kk + 4(g>>1) + e (+8), dv = 32d + 16(g&1) + 4c
  const int tr_g = lane >> 4, tr_e = (lane >> 2) & 3, tr_c = lane & 3;
  const int tr_row = 4 * (tr_g >> 1) + tr_e;
  uint32_t v_rd[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int chunk = 4 * d + 2 * (tr_g & 1) + (tr_c >> 1);
    v_rd[d] = V_OFF + tr_row * 256 + 16 * (chunk ^ (4 * tr_e)) + 8 * (tr_c & 1);
  }

  // ---- running softmax state (raw score units) and output accumulator O^T
  const float c = a.scale_log2;                      // |scale| * log2(e), > 0
  float m_run = -1e30f;                              // finite, so (m_old - m_new) stays defined
  float mc = m_run * c;
  float l_run = 0.f;                                 // this lane's share of the row sum
  bool fresh = true;                                 // no tile computed yet (wave-uniform)
  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x16{};

  // ---- prologue, ordered for the first tile's critical path: page ids first,
  // then the K_nope / V rows, then Q, so the K_rope loads wait for the page ids
  // only; the sign of a negative scale is applied to Q once it has arrived.
  uint32_t pg_next[2] = {0u, 0u};
  if (kt_hi > kt_lo) {
    const uint32_t pg0[2] = {page_of(kt_lo, 0), page_of(kt_lo, 1)};
    pg_next[0] = page_of(kt_lo + 1, 0);
    pg_next[1] = page_of(kt_lo + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    issue_kv(kt_lo, (MLA_LDS uint8_t*)lds + (kt_lo & 1) * STAGE);
    __builtin_amdgcn_sched_barrier(0);
    load_q();
    __builtin_amdgcn_sched_barrier(0);
    issue_rope(kt_lo, (MLA_LDS uint8_t*)lds + (kt_lo & 1) * STAGE, pg0);
  }
  // with no key to attend to, Q is never read (the epilogue writes 0, or passes
  // an earlier partial through)

  for (int32_t kt = kt_lo; kt < kt_hi; ++kt) {
    const int stage = kt & 1;
    // publish tile kt (every wave's loads done) and retire stage (kt+1)&1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt == kt_lo && a.scale < 0.f) {
#pragma unroll
      for (int ks = 0; ks < 12; ++ks)
        qop[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(i32x4, qop[ks]) ^ (int)0x80008000);
    }
    // The stage loaded here and the stage read below are the two disjoint halves
    // of the LDS buffer.  They reach the tile code as restrict pointers of one
    // inlined call, so the compiler can tell that reads of this tile do not depend
    // on the next tile's direct-to-LDS loads and does not wait for those (the
    // wait at the top of the next iteration and the barrier order them instead).
    auto step = [&](MLA_LDS uint8_t* __restrict__ ld, const MLA_LDS uint8_t* __restrict__ rd) {
    if (kt + 1 < kt_hi) {
      issue_kv(kt + 1, ld);
      issue_rope(kt + 1, ld, pg_next);
      pg_next[0] = page_of(kt + 2, 0);
      pg_next[1] = page_of(kt + 2, 1);
    }
    const int32_t j0 = kt * BN;
    // A wave whose last query comes before key 32 of the tile sees none of keys
    // 32..63 (key block 1): its S^T block, softmax terms and P.V steps for them
    // are skipped (they would add exact zeros), which saves their LDS reads.
    const bool half_tile = causal && c0 + j0 + 32 > wq_last;
    auto tile_body = [&](auto half_c) {
      constexpr bool HALF = decltype(half_c)::value;
      constexpr int KB = HALF ? 1 : 2;                 // key blocks of 32 this wave computes
      const MLA_LDS uint8_t* st = rd;
      // S^T = K Q^T.  K fragments go through a three-deep register ring, read two
      // k-steps ahead of their MFMAs so LDS latency overlaps the MFMA chain; the
      // scheduling barriers keep the compiler from sinking the reads to their uses.
      f32x16 s[2] = {f32x16{}, f32x16{}};
      bf16x8 kf[3][2];
      auto kread = [&](int ks, bf16x8 (&dst)[2]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const uint32_t off = ks < 8 ? kn_rd[ks] + kb * 32 * 256 : kr_rd[ks - 8] + kb * 32 * 128;
          dst[kb] = *reinterpret_cast<const MLA_LDS bf16x8*>(st + off);
        }
      };
      kread(0, kf[0]);
      kread(1, kf[1]);
      // The MFMA sections run at raised wave priority, so the other workgroup's
      // wave on this SIMD (in its softmax) yields the issue slot to MFMA issue.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) {
        if (ks + 2 < 12) kread(ks + 2, kf[(ks + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[kb] = mfma_bf16(kf[ks % 3][kb], qop[ks], s[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // s[kb][r] is key j0 + 32kb + 4hf + roff(r), roff(r) = 8(r/4) + r%4
      const bool full = (j0 + BN <= len) && (!causal || c0 + j0 + BN - 1 <= wq_first);
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int32_t kbase = j0 + 32 * kb + 4 * hf;
          const int32_t lim = causal ? min(len - 1 - kbase, p + my_i - c0 - kbase) : len - 1 - kbase;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int32_t roff = 8 * (r >> 2) + (r & 3);
            s[kb][r] = roff <= lim ? s[kb][r] : -INFINITY;
          }
        }
      }
      // first V fragments, read while the softmax runs
      bf16x8 vf[2][4];
      auto vread = [&](int kk, bf16x8 (&dst)[4]) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const MLA_LDS uint8_t* base = st + v_rd[d] + kk * 16 * 256;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(base));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4*)(base + 8 * 256));
          dst[d] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      };
      vread(0, vf[0]);
      asm volatile("" ::: "memory");   // keeps these reads ahead of the branches below
      // Weights p = exp2(s c - m c) against the running reference m.  The tile's
      // row max is taken only on the unit's first tile and when some lane's
      // weights leave the range the reference keeps them in (their sum above
      // WSUM_MAX, or not finite); then m moves to the max, O and l are
      // rescaled, and the weights are computed again (each is then at most 1).
      uint32_t pw[16];
      float ps = 0.f;
      auto weights = [&]() {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int x = 0; x < 8; ++x)
            pw[8 * kb + x] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * x], c, -mc)),
                                         __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * x + 1], c, -mc)));
        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int x = 0; x < 8 * KB; x += 2) {
          ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[x]), ones, ps0, false);
          ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[x + 1]), ones, ps1, false);
        }
        ps = ps0 + ps1;
      };
      bool redo = fresh;
      fresh = false;
      if (!redo) {
        weights();
        redo = __builtin_amdgcn_ballot_w64(!(ps <= WSUM_MAX)) != 0;
      }
      if (redo) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_across_halves(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        m_run = m_new;
        mc = m_run * c;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] *= alpha;
        weights();
      }
      l_run += ps;

      // O^T += V^T P^T, four (two) 16-key steps; V fragments are read one step ahead
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < 2 * KB; ++kk) {
        const i32x4 pv = {(int)pw[4 * kk], (int)pw[4 * kk + 1], (int)pw[4 * kk + 2], (int)pw[4 * kk + 3]};
        const bf16x8 pop = __builtin_bit_cast(bf16x8, pv);
        if (kk + 1 < 2 * KB) vread(kk + 1, vf[(kk + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = mfma_bf16(vf[kk & 1][d], pop, o[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    if (wave_rows && (!causal || c0 + j0 <= wq_last)) {
      if (half_tile)
        tile_body(std::true_type{});
      else
        tile_body(std::false_type{});
    }
    };
    // the stage is a constant in each copy of the tile code, so the LDS read
    // addresses take it as an immediate offset
    // (the key-split forms keep one copy: two exceed the register budget there)
    if constexpr (KVSPLIT)
      step((MLA_LDS uint8_t*)lds + (stage ^ 1) * STAGE, (const MLA_LDS uint8_t*)lds + stage * STAGE);
    else if (stage)
      step((MLA_LDS uint8_t*)lds, (const MLA_LDS uint8_t*)lds + STAGE);
    else
      step((MLA_LDS uint8_t*)lds + STAGE, (const MLA_LDS uint8_t*)lds);
  }

  // ---- epilogue: combine the two halves' row sums, normalise, store the row
  // with its log-sum-exp (merged with an earlier partial when one is given)
  const float l_tot = l_run + swap_halves(l_run);
  if constexpr (PLAIN && !KVSPLIT) {
    // Plain bf16 rows go through LDS (the stages are free once every wave is past
    // its last tile): row 32w + li of the tile, 16-byte chunk c at c ^ (row % 16).
    // Then 16 lanes store each query's whole 256-byte row with streaming stores,
    // which keep the output out of L2 (K/V tiles of other units are read there).
    // Storing the same 16-byte pieces straight from the registers with streaming
    // stores measured 1.7x slower on dsv3; this form measured 0.5-2 % faster than
    // plain stores from the registers.
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __syncthreads();
    MLA_LDS uint8_t* ot = (MLA_LDS uint8_t*)lds;
    const int row = 32 * w + li;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t w0 = pack_bf16x2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv);
        const uint32_t w1 = pack_bf16x2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv);
        *reinterpret_cast<MLA_LDS u32x2*>(ot + row * 256 + 16 * ((4 * d + g) ^ (row & 15)) + 8 * hf) =
            u32x2{w0, w1};
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = 16 * it + (tid >> 4), cc = tid & 15;
      if ((int32_t)i0 + r < (int32_t)n) {
        const i32x4 v = *reinterpret_cast<const MLA_LDS i32x4*>(ot + r * 256 + 16 * (cc ^ (r & 15)));
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
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? mc + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    if (KVSPLIT && part)
      store_output_row<false>(kv_split_target(a, (u.qt & 1u) ^ 1u), (size_t)(t0 + my_i) * H + h, hf, o, inv, lse2);
    else
      store_output_row<PLAIN>(row_target(a, row_first, row_last), (size_t)(t0 + my_i) * H + h, hf, o, inv, lse2);
  }
}

hipError_t launch_prefill_bf16(PrefillArgs a, uint32_t q_max, hipStream_t stream) {
  a.qtiles = (q_max + BM - 1) / BM;
  const bool kv_split = a.split_keys != 0;
  const uint64_t units = (uint64_t)a.heads * a.batch * a.qtiles * (kv_split ? 2u : 1u);
  const uint64_t grid = (units + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  const bool plain = !a.out_fp32 && !a.lse && !a.prev_out && !a.row_mode;
  if (kv_split) {
    // full query, no row mode, no earlier partial (the entry point checks)
    auto kernel = a.causal ? (plain ? prefill_bf16_kernel<true, true, false, true> : prefill_bf16_kernel<true, false, false, true>)
                           : (plain ? prefill_bf16_kernel<false, true, false, true> : prefill_bf16_kernel<false, false, false, true>);
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(NT), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_kv_split_merge(a, stream);
  }
  auto kernel = a.q_split
      ? (a.causal ? (plain ? prefill_bf16_kernel<true, true, true, false> : prefill_bf16_kernel<true, false, true, false>)
                  : (plain ? prefill_bf16_kernel<false, true, true, false> : prefill_bf16_kernel<false, false, true, false>))
      : (a.causal ? (plain ? prefill_bf16_kernel<true, true, false, false> : prefill_bf16_kernel<true, false, false, false>)
                  : (plain ? prefill_bf16_kernel<false, true, false, false> : prefill_bf16_kernel<false, false, false, false>));
  hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
