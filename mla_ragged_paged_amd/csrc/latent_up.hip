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
// W rows as the A operand and the gathered latent rows as B.  A workgroup of
// eight waves owns 256 output features (one head: its 128 key rows and 128
// value rows) x 256 buffer slots, so every weight and latent row it stages
// serves 256 outputs and the L2 -> LDS traffic is 1/128 byte per FLOP (a
// 128 x 128 tile, measured at 15-20 % lower throughput, moves twice that).  Each wave owns
// 128 features x 64 slots (4 x 2 MFMA tiles, 128 accumulator VGPRs).  The
// reduction runs in chunks of 64 latent columns through two LDS stages of
// 64 KB (weights 32 KB, latent 32 KB), filled by direct-to-LDS buffer loads:
// weight rows by plain offsets, latent rows through the page table (each lane
// resolves its four slots' cache rows once, from the plan row kept in LDS).
// 16-byte chunks are XOR-swizzled by (row / 2) % 8, which keeps the operand
// reads free of bank conflicts; operand fragments are read one k-step ahead of
// their MFMAs.  The epilogue rounds to bf16, transposes through LDS and writes
// whole 256-byte rows of K_nope and V.
#include "device_common.h"
#include "kernels.h"

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
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LLDS];

  // ---- tile.  XCD x (workgroup id % 8) takes a contiguous eighth of the heads.
  // Within it, tiles run in blocks of up to 8 heads x 8 slot tiles (head
  // fastest), so the 32 workgroups an XCD runs at once share 2 MB of weight rows
  // and 2 MB of latent rows, both held by its 4 MB L2.
  const uint32_t nt = a.heads;                     // feature tiles: one per head
  const uint32_t mtn = (a.cap + TS - 1) / TS;      // slot tiles
  const uint32_t bid = blockIdx.x;
  uint32_t ft, mt;
  {
    const bool split8 = (nt & 7u) == 0;
    const uint32_t per = split8 ? nt >> 3 : nt;
    const uint32_t f_base = split8 ? (bid & 7u) * per : 0u;
    const uint32_t j = split8 ? bid >> 3 : bid;
    const uint32_t gf = min(per, 8u), gm = 8u;
    const uint32_t mg = j / (per * gm);
    const uint32_t r = j - mg * per * gm;
    const uint32_t gml = min(gm, mtn - mg * gm);
    const uint32_t fg = r / (gf * gml);
    const uint32_t gfl = min(gf, per - fg * gf);
    const uint32_t q = r - fg * gf * gml;
    ft = f_base + fg * gf + q % gfl;
    mt = mg * gm + q / gfl;
  }
  const uint32_t used = a.bro[a.batch];            // slots this plan row fills
  const uint32_t m0 = mt * TS;
  if (m0 >= used) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int li = lane & 31, hf = lane >> 5;

  // ---- the plan row in LDS, then each lane's four latent rows (slot
  // m0 + 32w + 8u + lane/8 for load u) as byte offsets into the cache layer
  uint32_t* sbro = reinterpret_cast<uint32_t*>(lds);
  for (uint32_t i = tid; i <= a.batch; i += NTH) sbro[i] = a.bro[i];
  __syncthreads();
  uint32_t row_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t g = m0 + 32 * w + 8 * u + (lane >> 3);
    row_off[u] = a.cache_bytes;                     // past the end: the load returns zeros
    if (g < used && g >= sbro[0]) {
      uint32_t lo = 0, hi = a.batch;                // last b with sbro[b] <= g, b < batch
      while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (sbro[mid] <= g) lo = mid; else hi = mid;
      }
      const uint32_t pos = a.co[lo] + (g - sbro[lo]);
      const uint32_t* pt = a.page_table + (size_t)lo * a.max_pages;
      const uint32_t page = a.page_shift < 32u ? pt[pos >> a.page_shift] : pt[pos / a.page_size];
      const uint32_t slot = a.page_shift < 32u ? (pos & (a.page_size - 1u)) : (pos % a.page_size);
      row_off[u] = (page * a.page_size + slot) * a.row_bytes + a.latent_col * 2;
    }
  }
  __syncthreads();                                  // the plan row's LDS is reused below

  // ---- load slots: load u of wave w covers tile rows 32w + 8u .. +7; lane ->
  // row 32w + 8u + lane/8, stored chunk lane%8 holds source chunk (lane%8) ^ swz(row)
  const uint32_t n0 = ft * TF;
  const uint32_t kdim = a.latent_dim;
  const auto w_rs = rsrc(a.w + (size_t)n0 * kdim, TF * kdim * 2);
  const auto c_rs = rsrc(a.cache, a.cache_bytes);
  uint32_t a_off[4], b_src[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 32 * w + 8 * u + (lane >> 3);
    const uint32_t cs = (uint32_t)((lane & 7) ^ swz(r));
    a_off[u] = (uint32_t)r * kdim * 2 + 16u * cs;
    b_src[u] = row_off[u] + 16u * cs;
  }
  auto issue = [&](uint32_t kc, int stage) {
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

  f32x16 acc[4][2];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};

  const uint32_t nkc = kdim / KC;
  issue(0, 0);
  for (uint32_t kc = 0; kc < nkc; ++kc) {
    const int stage = kc & 1;
    // publish chunk kc (every wave's loads done) and retire the other stage
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kc + 1 < nkc) issue(kc + 1, stage ^ 1);
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
  }

  // ---- epilogue: acc[x][y][i] is feature 128wn + 32x + 8(i/4) + 4hf + i%4 of
  // slot 64wm + 32y + li.  Round to bf16 and write the tile as [slot][feature]
  // (512 B per slot: key 256 B then value 256 B; 16-byte chunk c at c ^ (slot % 32)),
  // then store whole rows.
  __syncthreads();                                  // every wave is done reading the stages
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
  const uint32_t head = ft;
  const size_t row_stride = (size_t)a.heads * 128;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int r = 16 * it + (tid >> 5), c = tid & 31;    // 32 chunks per slot: 16 key + 16 value
    const uint32_t g = m0 + r;
    if (g < used) {
      const i32x4 val = *reinterpret_cast<const MLA_LDS i32x4*>((MLA_LDS uint8_t*)lds + r * 512 + 16 * (c ^ (r & 31)));
      uint16_t* dst = (c < 16 ? a.k_nope : a.v) + g * row_stride + head * 128 + (c & 15) * 8;
      st16(dst, val);
    }
  }
}

}  // namespace

hipError_t launch_latent_up(const LatentArgs& a, hipStream_t stream) {
  const uint64_t mt = (a.cap + TS - 1) / TS;
  const uint64_t grid = mt * a.heads;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(latent_up_kernel, dim3((uint32_t)grid), dim3(NTH), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
