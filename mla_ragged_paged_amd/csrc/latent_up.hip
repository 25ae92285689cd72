// Latent up-projection: per-head K_nope and V of one buffer row, computed
// straight from the paged latent cache.  The pages describe a latent cache
// (page "mla_prefill_v2_ragged", Args: the V operand is the nope segment of the
// latent cache) and the plan whose rows say which cache positions fill which
// buffer slots (page "generic_flare_mla_prefill_ragged_paged_plan",
// description and Args); the decompression itself is the DeepSeek-V2/V3 one:
//   K_nope[g][h][d] = sum_c W[h*256 + d][c]       * c_g[c]
//   V[g][h][d]      = sum_c W[h*256 + 128 + d][c] * c_g[c]
// with c_g the latent (a column window of the cache row) of the position that
// slot g holds, and W [H*256][latent_dim] bf16.
//
// A dense contraction, so it runs on the 32x32x16 bf16 MFMA: C^T = W . L^T with
// W rows as the A operand and the gathered latent rows as B.  A tile is 256
// output features (one head: its 128 key rows and 128 value rows) x 256 buffer
// slots, so every weight and latent row staged serves 256 outputs and the
// L2 -> LDS traffic is 1/128 byte per FLOP (a 128 x 128 tile, measured at 15-20 %
// lower throughput, moves twice that).  A workgroup of eight waves computes one
// tile at a time; each wave owns 128 features x 64 slots (4 x 2 MFMA tiles, 128
// accumulator VGPRs).  The reduction runs in chunks of 64 latent columns through
// two LDS stages of 64 KB (weights 32 KB, latent 32 KB), filled by
// direct-to-LDS buffer loads: weight rows by plain offsets, latent rows through
// the page table (each lane resolves its four slots' cache rows from the plan
// row, which stays in LDS for the whole launch).  16-byte chunks are
// XOR-swizzled by (row / 2) % 8, which keeps the operand reads free of bank
// conflicts; operand fragments are read one k-step ahead of their MFMAs.
//
// The grid is persistent: one workgroup per CU (the 160 KB of LDS allow no
// more) takes its XCD's tiles in turn.  The next tile's latent rows are looked
// up while the current tile's first chunk runs, and its first chunk is loaded
// as soon as the epilogue has handed the stage memory back, so a tile starts
// without a cold page-table lookup or a workgroup launch.  The epilogue rounds
// to bf16, transposes through LDS and writes whole 256-byte rows of K_nope and V
// with streaming (non-temporal) stores: the rows are not read again by this
// kernel, and keeping them out of L2 leaves it to the weight and latent rows
// (measured 13-15 % faster than plain stores on the 16K-token and prefix rows).
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "mla_prefill.h"

namespace mla {
namespace {

constexpr int TF = 256;               // features per tile (one head: 128 key + 128 value rows)
constexpr int TS = 256;               // slots per tile
constexpr int KC = 64;                // latent columns per chunk
constexpr int NTH = 512;              // 8 waves
constexpr int A_OFF = 0;              // W tile      [256 rows][8 chunks of 16 B] 32 KiB
constexpr int B_OFF = TF * KC * 2;    // latent tile [256 rows][8 chunks]          32 KiB
constexpr int LSTAGE = (TF + TS) * KC * 2;   // 64 KiB
constexpr int LLDS = 2 * LSTAGE;             // 128 KiB
constexpr int PLAN_BYTES = 4 * MLA_MAX_BATCH;       // plan row entries [0, batch): 32 KiB

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bload_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, MLA_LDS void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ void __launch_bounds__(NTH, 1) latent_up_kernel(LatentArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LLDS + PLAN_BYTES];
  uint32_t* sbro = reinterpret_cast<uint32_t*>(lds + LLDS);    // plan row, entries [0, batch)

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, hf = lane >> 5;

  // ---- this workgroup's tiles.  With H a multiple of 8, XCD x (workgroup id % 8)
  // owns the tiles of heads [x*H/8, (x+1)*H/8) and its workgroups take that list
  // round-robin; the list runs in blocks of up to 4 heads x 8 slot tiles (head
  // fastest), so the 32 tiles an XCD runs at once share 1 MB of weight rows and
  // 2 MB of latent rows, both held by its 4 MB L2 (blocks of 8 heads, 4 MB in
  // all, measured 1-2 % slower).
  const uint32_t used = min(a.bro[a.batch], a.cap);   // slots this plan row fills
  const uint32_t mtn = (used + TS - 1) / TS;       // slot tiles holding a used slot
  const bool split8 = (a.heads & 7u) == 0;
  const uint32_t per = split8 ? a.heads >> 3 : a.heads;
  const uint32_t f_base = split8 ? (blockIdx.x & 7u) * per : 0u;
  const uint32_t wgs = split8 ? gridDim.x >> 3 : gridDim.x;
  const uint32_t ntiles = per * mtn;
  auto tile_of = [&](uint32_t j, uint32_t& ft, uint32_t& mt) {
    const uint32_t gf = min(per, 4u), gm = 8u;
    const uint32_t mg = j / (per * gm);
    const uint32_t r = j - mg * per * gm;
    const uint32_t gml = min(gm, mtn - mg * gm);
    const uint32_t fg = r / (gf * gml);
    const uint32_t gfl = min(gf, per - fg * gf);
    const uint32_t q = r - fg * gf * gml;
    ft = f_base + fg * gf + q % gfl;
    mt = mg * gm + q / gfl;
  };
  uint32_t j = split8 ? blockIdx.x >> 3 : blockIdx.x;
  if (j >= ntiles) return;

  for (uint32_t i = tid; i < a.batch; i += NTH) sbro[i] = a.bro[i];
  __syncthreads();

  // each lane's four latent rows of slot tile mt (slot 32w + 8u + lane/8 for
  // load u) as byte offsets into the cache layer; the source chunk is folded in
  auto rows_of = [&](uint32_t mt, uint32_t (&src)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 32 * w + 8 * u + (lane >> 3);
      const uint32_t g = mt * TS + (uint32_t)r;
      uint32_t off = a.cache_bytes;                 // past the end: the load returns zeros
      if (g < used && g >= sbro[0]) {
        uint32_t lo = 0, hi = a.batch;              // last b with sbro[b] <= g, b < batch
        while (hi - lo > 1) {
          const uint32_t mid = (lo + hi) >> 1;
          if (sbro[mid] <= g) lo = mid; else hi = mid;
        }
        const uint32_t pos = a.co[lo] + (g - sbro[lo]);
        const uint32_t* pt = a.page_table + (size_t)lo * a.max_pages;
        const uint32_t page = a.page_shift < 32u ? pt[pos >> a.page_shift] : pt[pos / a.page_size];
        const uint32_t slot = a.page_shift < 32u ? (pos & (a.page_size - 1u)) : (pos % a.page_size);
        off = (page * a.page_size + slot) * a.row_bytes + a.latent_col * 2;
      }
      src[u] = off + 16u * (uint32_t)((lane & 7) ^ swz(r));
    }
  };

  // ---- load slots: load u of wave w covers tile rows 32w + 8u .. +7; lane ->
  // row 32w + 8u + lane/8, stored chunk lane%8 holds source chunk (lane%8) ^ swz(row)
  const uint32_t kdim = a.latent_dim;
  const auto c_rs = rsrc(a.cache, a.cache_bytes);
  uint32_t a_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 32 * w + 8 * u + (lane >> 3);
    a_off[u] = (uint32_t)r * kdim * 2 + 16u * (uint32_t)((lane & 7) ^ swz(r));
  }
  auto w_rsrc = [&](uint32_t ft) { return rsrc(a.w + (size_t)ft * TF * kdim, TF * kdim * 2); };
  auto issue = [&](__amdgpu_buffer_rsrc_t w_rs, const uint32_t (&b_src)[4], uint32_t kc, int stage) {
    MLA_LDS uint8_t* st = (MLA_LDS uint8_t*)lds + stage * LSTAGE;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int m = 4 * w + u;
      bload_lds(w_rs, a_off[u] + kc * (KC * 2), st + A_OFF + m * 1024);
      bload_lds(c_rs, b_src[u] + kc * (KC * 2), st + B_OFF + m * 1024);
    }
  };

  // ---- operand reads: wave (wn, wm) = (w & 1, w >> 1) owns features
  // 128wn .. +127 and slots 64wm .. +63; fragment x of k-step ks is row
  // base + 32x + li, columns 16ks + 8hf .. +7
  const int wn = w & 1, wm = w >> 1;
  uint32_t a_rd[4][4], b_rd[2][4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int ra = 128 * wn + 32 * x + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a_rd[x][ks] = A_OFF + ra * 128 + 16 * ((2 * ks + hf) ^ swz(ra));
  }
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int rb = 64 * wm + 32 * y + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) b_rd[y][ks] = B_OFF + rb * 128 + 16 * ((2 * ks + hf) ^ swz(rb));
  }

  // ---- tiles in turn.  Each tile's chunks go through stages 0, 1, 0, ...; the
  // next tile's latent rows are looked up while the first chunk runs.
  const uint32_t nkc = kdim / KC;
  uint32_t ft, mt;
  tile_of(j, ft, mt);
  uint32_t b_src[4];
  rows_of(mt, b_src);
  auto w_rs = w_rsrc(ft);
  issue(w_rs, b_src, 0, 0);
  int stage = 0;
  const size_t row_stride = (size_t)a.heads * 128;
  while (true) {
    const uint32_t jn = j + wgs;
    const bool more = jn < ntiles;
    uint32_t ftn = 0, mtn_ = 0;
    uint32_t b_next[4] = {0u, 0u, 0u, 0u};
    f32x16 acc[4][2];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
    for (uint32_t kc = 0; kc < nkc; ++kc) {
      // publish chunk kc (every wave's loads done) and retire the other stage
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kc == 0 && more) {
        tile_of(jn, ftn, mtn_);
        rows_of(mtn_, b_next);
      }
      if (kc + 1 < nkc) issue(w_rs, b_src, kc + 1, stage ^ 1);
      const uint8_t* st = lds + stage * LSTAGE;
      // fragments of k-step ks + 1 are read while the MFMAs of ks run
      bf16x8 fa[2][4], fb[2][2];
      auto rd = [&](int ks, int slot) {
#pragma unroll
        for (int x = 0; x < 4; ++x) fa[slot][x] = *reinterpret_cast<const bf16x8*>(st + a_rd[x][ks]);
#pragma unroll
        for (int y = 0; y < 2; ++y) fb[slot][y] = *reinterpret_cast<const bf16x8*>(st + b_rd[y][ks]);
      };
      rd(0, 0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks + 1 < 4) rd(ks + 1, (ks + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y) acc[x][y] = mfma_bf16(fa[ks & 1][x], fb[ks & 1][y], acc[x][y]);
        __builtin_amdgcn_sched_barrier(0);
      }
      stage ^= 1;
    }

    // ---- epilogue: acc[x][y][i] is feature 128wn + 32x + 8(i/4) + 4hf + i%4 of
    // slot 64wm + 32y + li.  Round to bf16 and write the tile as [slot][feature]
    // (512 B per slot: key 256 B then value 256 B; 16-byte chunk c at c ^ (slot % 32))
    // through the stage memory, take each thread's 16 row chunks back into
    // registers, hand the memory to the next tile's first loads, then store whole
    // rows (streaming stores: the rows are not read again here).
    __syncthreads();                                // every wave is done reading the stages
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const int r = 64 * wm + 32 * y + li;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = 128 * wn + 32 * x + 8 * q + 4 * hf;
          const uint32_t w0 = pack_bf16x2(acc[x][y][4 * q], acc[x][y][4 * q + 1]);
          const uint32_t w1 = pack_bf16x2(acc[x][y][4 * q + 2], acc[x][y][4 * q + 3]);
          const int chunk = (f >> 3) ^ (r & 31);
          *reinterpret_cast<MLA_LDS u32x2*>((MLA_LDS uint8_t*)lds + r * 512 + 16 * chunk + 2 * (f & 7)) =
              u32x2{w0, w1};
        }
      }
    __syncthreads();
    i32x4 rowv[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int r = 16 * it + (tid >> 5), cc = tid & 31;
      rowv[it] = *reinterpret_cast<const MLA_LDS i32x4*>((MLA_LDS uint8_t*)lds + r * 512 + 16 * (cc ^ (r & 31)));
    }
    __syncthreads();                                // the stage memory is free again
    if (more) issue(w_rsrc(ftn), b_next, 0, 0);
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int r = 16 * it + (tid >> 5), cc = tid & 31;
      const uint32_t g = mt * TS + r;
      if (g < used) {
        uint16_t* dst = (cc < 16 ? a.k_nope : a.v) + g * row_stride + ft * 128 + (cc & 15) * 8;
        __builtin_nontemporal_store(rowv[it], reinterpret_cast<i32x4*>(dst));
      }
    }
    if (!more) break;
    stage = 0;
    j = jn;
    ft = ftn;
    mt = mtn_;
    w_rs = w_rsrc(ft);
#pragma unroll
    for (int u = 0; u < 4; ++u) b_src[u] = b_next[u];
  }
}

}  // namespace

hipError_t launch_latent_up(const LatentArgs& a, hipStream_t stream) {
  // one workgroup per CU at most (256 CUs, 32 per XCD), each taking tiles in turn
  const uint64_t tiles = (uint64_t)(a.cap + TS - 1) / TS * a.heads;
  if (tiles == 0) return hipSuccess;
  const uint64_t grid = (a.heads & 7u) == 0 ? 8u * std::min<uint64_t>(32u, tiles / 8u) : std::min<uint64_t>(256u, tiles);
  hipLaunchKernelGGL(latent_up_kernel, dim3((uint32_t)grid), dim3(NTH), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
