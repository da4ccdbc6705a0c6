// bf16 "TN" GEMM on gfx950 MFMA: C[m, n] = A[m, k] * B[n, k]^T, fp32 accumulate.
//
// Used for every projection of an SPTS layer (K/V over all candidates, Q of
// the probe and selected rows, the O projection, the LTP proxy products and
// the reduced SwiGLU FFN).  Both operands are k-contiguous, so a wave reads
// each MFMA fragment as one 16-byte LDS load.
//
// Tiling: 256 x 256 x 64 per workgroup, 8 waves in a 4 (M) x 2 (N) grid, each
// wave owns a 64 x 128 block = 2 x 4 tiles of v_mfma_f32_32x32x16_bf16 (128
// fp32 accumulators per lane), two waves per SIMD.  Operands go straight from
// global memory into double-buffered LDS (2 x 64 KiB), one barrier per
// k-step.  Only waves 0-3 (one per SIMD) issue the global->LDS loads: a wave
// stalled on issuing them cannot issue MFMAs, so each SIMD keeps one wave
// that only computes.
//
// The MFMA is issued as (B fragment, A fragment) so each lane's accumulators
// hold ONE row of C and 4 groups of 4 consecutive columns; every epilogue
// (row scatter, RoPE pairs, SwiGLU pairs, row norms) is then lane-local.
#include <atomic>
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"

namespace spts {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 512;
constexpr int TILE_ELEMS = BM * BK;  // per operand per stage

// Element offset in a 64-wide (128-byte-row) LDS tile.  gfx950 serves a
// 16-byte-per-lane LDS read 16 lanes at a time across 64 banks (256 bytes), so
// the 16 rows read together must land in 16 distinct 16-byte slots: rows of
// equal parity share a 128-byte half, and XOR-ing the chunk with (row >> 1)
// spreads each half's 8 rows over its 8 slots.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

template <int EPI, bool GATHER>
__global__ __launch_bounds__(NTHREADS, 1)
void gemm_tn_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* As = smem;                       // [2][BM*BK]
  uint16_t* Bs = smem + 2 * TILE_ELEMS;      // [2][BN*BK]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS addresses in SGPRs
  const int wm = wave >> 1, wn = wave & 1;          // 4 x 2 waves
  const int l32 = lane & 31, half = lane >> 5;

  // ---- tile order.  Workgroups are dealt round-robin to the 8 XCDs, so
  // workgroup b runs on XCD b % 8.  Each XCD gets a contiguous run of the
  // logical tile order, and that order walks groups of GROUP_M row tiles
  // across all column tiles, so the ~32 tiles resident on one XCD at a time
  // form a 4 x 8 block that shares A and B k-slices in that XCD's L2.
  const int tiles_m = (g.m + BM - 1) / BM;
  constexpr bool kSwiglu = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SPLIT);
  const int tiles_n = kSwiglu ? (g.n / 2) / 128 : g.n / BN;
  const int ksplit = (EPI == EPI_PARTIAL) ? g.ksplit : 1;
  const int total = tiles_m * tiles_n * ksplit;
  const int per_xcd = (total + 7) / 8;
  const int logical_k = ((int)blockIdx.x & 7) * per_xcd + ((int)blockIdx.x >> 3);
  if (logical_k >= total) return;                     // padding workgroups of the last XCD run
  const int kslice = logical_k % ksplit;              // split-K slice (0 without split)
  const int logical = logical_k / ksplit;
  constexpr int GROUP_M = 4;
  const int in_group = GROUP_M * tiles_n;
  const int first_m = (logical / in_group) * GROUP_M;
  const int gm = min(GROUP_M, tiles_m - first_m);
  const int tile_m = first_m + (logical % in_group) % gm;
  const int tile_n = (logical % in_group) / gm;

  // KV: tiles at or past column n0 read b1 and write out2
  const bool part1 = (EPI == EPI_KV) && tile_n * BN >= g.n0;

  // ---- direct global -> LDS staging by waves 0-3.  Loading wave w,
  // instruction i writes the 1 KiB block of tile rows rb*8 .. rb*8+7,
  // rb = 4*i + w; lane L lands at row r = rb*8 + L/8, physical chunk L%8, so
  // it fetches the logical chunk (L%8) ^ ((r >> 1) & 7) -- the swizzle of
  // swz() applied on the global side.
  const bool loader = wave < 4;
  const int lw = wave & 3;
  const int ld_sub = lane >> 3;                       // row within the 8-row block
  uint32_t a_off[8], b_off[8];                        // byte offsets of the staged rows
  unsigned b_from_up = 0;                             // SWIGLU: instruction i reads Wu
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rb = 4 * i + lw;
    const int r = rb * 8 + ld_sub;                    // row within the 256-row tile
    const int ld_ch = (lane & 7) ^ ((r >> 1) & 7);    // logical 16-byte chunk fetched
    int ar = tile_m * BM + r;
    if (ar >= g.m) ar = g.m - 1;
    if (GATHER) ar = g.a_rows[ar];
    a_off[i] = ((uint32_t)ar * (uint32_t)g.lda + ld_ch * 8) * 2u;
    if (kSwiglu) {
      // wave column block r / 128: rows 0..63 gate, 64..127 up, same 64 outputs
      const int within = r & 127;
      const uint32_t brow = (uint32_t)tile_n * 128 + (r >> 7) * 64 + (within & 63);
      if (within >= 64) b_from_up |= 1u << i;
      b_off[i] = (brow * (uint32_t)g.ldb + ld_ch * 8) * 2u;
    } else {
      const uint32_t brow = (uint32_t)(tile_n * BN - (part1 ? g.n0 : 0)) + r;
      b_off[i] = (brow * (uint32_t)g.ldb + ld_ch * 8) * 2u;
    }
  }
  const char* abase = reinterpret_cast<const char*>(g.a);
  const char* b0base = reinterpret_cast<const char*>(part1 ? g.b1 : g.b0);
  const char* b1base = reinterpret_cast<const char*>(g.b1);
  const int KT = g.k / BK / ksplit;                    // k-steps of this slice
  const int kt_base = kslice * KT;

  auto issue = [&](int kt_local, int stage) {
    if (!loader) return;
    const int kt = kt_base + kt_local;
    const uint32_t ka = (uint32_t)kt * BK * 2u;
    const uint32_t kb = (g.kwrap > 0 ? (uint32_t)((kt * BK) % g.kwrap) : (uint32_t)kt * BK) * 2u;
    uint16_t* a_s = As + stage * TILE_ELEMS;
    uint16_t* b_s = Bs + stage * TILE_ELEMS;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rb = 4 * i + lw;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(abase + a_off[i] + ka),
          (__attribute__((address_space(3))) void*)(a_s + rb * 512), 16, 0, 0);
      const char* bb = (kSwiglu && ((b_from_up >> i) & 1u)) ? b1base : b0base;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(bb + b_off[i] + kb),
          (__attribute__((address_space(3))) void*)(b_s + rb * 512), 16, 0, 0);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // k-step kt reads stage kt & 1 while the loads of k-step kt+1 fill the
  // other stage; the wait + barrier at its end hands both stages over.
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    // the last k-step reloads its own tile into the idle stage (never read)
    issue(kt + 1 < KT ? kt + 1 : kt, cur ^ 1);
    const uint16_t* a_s = As + cur * TILE_ELEMS;
    const uint16_t* b_s = Bs + cur * TILE_ELEMS;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + half;
      bf16x8 af[2], bfm[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(a_s + swz(wm * 64 + i * 32 + l32, ch));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfm[j] = *reinterpret_cast<const bf16x8*>(b_s + swz(wn * 128 + j * 32 + l32, ch));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(bfm[j], af[i], acc[i][j]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogues
  // lane holds C[row][col] for row = tile_m*BM + wm*64 + i*32 + l32 and
  // col = (tile base) + wn*128 + j*32 + q*8 + half*4 + e, r = q*4 + e.
  if (EPI == EPI_PARTIAL) {
    float* part = g.partial + (long)kslice * g.m * g.n;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = tile_m * BM + wm * 64 + i * 32 + l32;
      if (row >= g.m) continue;
      float* prow = part + (long)row * g.n;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = tile_n * BN + wn * 128 + j * 32 + q * 8 + half * 4;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][q * 4 + e];
          *reinterpret_cast<f32x4*>(prow + col) = v;
        }
    }
    return;
  }
  if (EPI == EPI_SUMSQ) {
    float* red = reinterpret_cast<float*>(smem);   // [4 wm][2 i][32 rows] from wn == 1
    float ss[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float t = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) t += acc[i][j][r] * acc[i][j][r];
      t += __shfl_xor(t, 32);
      ss[i] = t;
    }
    if (wn == 1 && half == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) red[(wm * 2 + i) * 32 + l32] = ss[i];
    }
    __syncthreads();
    if (wn == 0 && half == 0) {
      float* out = reinterpret_cast<float*>(g.out);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = tile_m * BM + wm * 64 + i * 32 + l32;
        if (row < g.m) out[(long)row * tiles_n + tile_n] = ss[i] + red[(wm * 2 + i) * 32 + l32];
      }
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = tile_m * BM + wm * 64 + i * 32 + l32;
    if (row >= g.m) continue;
    if (kSwiglu) {
      uint16_t* out = reinterpret_cast<uint16_t*>(g.out) + (long)row * g.ldc;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gt = acc[i][j][q * 4 + e];
            const float up = acc[i][j + 2][q * 4 + e];
            hv[e] = (gt / (1.0f + __expf(-gt))) * up;
          }
          const int col = tile_n * 128 + wn * 64 + j * 32 + q * 8 + half * 4;
          u32x2 w;
          w[0] = pack2bf(hv[0], hv[1]);
          w[1] = pack2bf(hv[2], hv[3]);
          *reinterpret_cast<u32x2*>(out + col) = w;
          if (EPI == EPI_SWIGLU_SPLIT) {
            u32x2 wl;
            wl[0] = pack2bf(hv[0] - lo_bf(w[0]), hv[1] - hi_bf(w[0]));
            wl[1] = pack2bf(hv[2] - lo_bf(w[1]), hv[3] - hi_bf(w[1]));
            *reinterpret_cast<u32x2*>(out + g.n / 2 + col) = wl;
          }
        }
      continue;
    }
    if (EPI == EPI_SPLIT) {
      uint16_t* out = reinterpret_cast<uint16_t*>(g.out) + (long)row * g.ldc;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float hi[4], lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t = acc[i][j][q * 4 + e];
            hi[e] = bf2f(f2bf(t));
            lo[e] = t - hi[e];
          }
          const int col = tile_n * BN + wn * 128 + j * 32 + q * 8 + half * 4;
          u32x2 wh, wl;
          wh[0] = pack2bf(hi[0], hi[1]); wh[1] = pack2bf(hi[2], hi[3]);
          wl[0] = pack2bf(lo[0], lo[1]); wl[1] = pack2bf(lo[2], lo[3]);
          *reinterpret_cast<u32x2*>(out + col) = wh;
          *reinterpret_cast<u32x2*>(out + g.n + col) = wl;
        }
      continue;
    }
    if (EPI == EPI_ROPE || (EPI == EPI_KV && !part1 && g.rope_table)) {
      const int arow = GATHER ? g.a_rows[row] : row;
      const float* tab = g.rope_table + (long)g.pos[arow] * 128;   // 64 (cos, sin) pairs
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = j * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
          const float cs = tab[2 * c], sn = tab[2 * c + 1];
          const float x1 = acc[i][j][r], x2 = acc[i][j + 2][r];
          acc[i][j][r] = x1 * cs - x2 * sn;
          acc[i][j + 2][r] = x2 * cs + x1 * sn;
        }
    }
    // EPI_STORE / EPI_ROPE / EPI_KV
    const int orow = g.out_rows ? g.out_rows[row] : row;
    uint16_t* out = part1 ? reinterpret_cast<uint16_t*>(g.out2) + (long)orow * g.ldc2
                          : reinterpret_cast<uint16_t*>(g.out) + (long)orow * g.ldc;
    const int cshift = part1 ? g.n0 : 0;                  // KV: b1 columns restart at 0
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = tile_n * BN + wn * 128 + j * 32 + q * 8 + half * 4 - cshift;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][q * 4 + e];
        u32x2 w;
        if (g.accumulate) {
          const u32x2 old = *reinterpret_cast<const u32x2*>(out + col);
          // the projection result is rounded to bf16 before the residual add
          w[0] = pack2bf(lo_bf(old[0]) + bf2f(f2bf(v[0])), hi_bf(old[0]) + bf2f(f2bf(v[1])));
          w[1] = pack2bf(lo_bf(old[1]) + bf2f(f2bf(v[2])), hi_bf(old[1]) + bf2f(f2bf(v[3])));
        } else {
          w[0] = pack2bf(v[0], v[1]);
          w[1] = pack2bf(v[2], v[3]);
        }
        *reinterpret_cast<u32x2*>(out + col) = w;
      }
  }
}

// Split-K finish: sum the fp32 slices in slice order and apply the epilogue.
// Thread = (row, 4-column group); for RoPE only groups in the first half of
// a 128-wide head work, each handling its pair group c+64.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs g) {
  const long groups = (long)g.m * (g.n / 4);
  for (long u = (long)blockIdx.x * blockDim.x + threadIdx.x; u < groups; u += (long)gridDim.x * blockDim.x) {
    const int row = (int)(u / (g.n / 4));
    const int col = (int)(u % (g.n / 4)) * 4;
    if (EPI == EPI_ROPE && (col & 127) >= 64) continue;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < g.ksplit; ++ks) {
      const float* prow = g.partial + ((long)ks * g.m + row) * g.n;
      a += *reinterpret_cast<const f32x4*>(prow + col);
      if (EPI == EPI_ROPE) b += *reinterpret_cast<const f32x4*>(prow + col + 64);
    }
    if (EPI == EPI_ROPE) {
      const int arow = g.a_rows ? g.a_rows[row] : row;
      const float* tab = g.rope_table + (long)g.pos[arow] * 128;
      const int c0 = col & 127;
      f32x4 y1, y2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float cs = tab[2 * (c0 + e)], sn = tab[2 * (c0 + e) + 1];
        y1[e] = a[e] * cs - b[e] * sn;
        y2[e] = b[e] * cs + a[e] * sn;
      }
      uint16_t* out = reinterpret_cast<uint16_t*>(g.out) + (long)row * g.ldc;
      u32x2 w1, w2;
      w1[0] = pack2bf(y1[0], y1[1]); w1[1] = pack2bf(y1[2], y1[3]);
      w2[0] = pack2bf(y2[0], y2[1]); w2[1] = pack2bf(y2[2], y2[3]);
      *reinterpret_cast<u32x2*>(out + col) = w1;
      *reinterpret_cast<u32x2*>(out + col + 64) = w2;
    } else if (EPI == EPI_SPLIT) {
      uint16_t* out = reinterpret_cast<uint16_t*>(g.out) + (long)row * g.ldc;
      float hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = bf2f(f2bf(a[e]));
        lo[e] = a[e] - hi[e];
      }
      u32x2 wh, wl;
      wh[0] = pack2bf(hi[0], hi[1]); wh[1] = pack2bf(hi[2], hi[3]);
      wl[0] = pack2bf(lo[0], lo[1]); wl[1] = pack2bf(lo[2], lo[3]);
      *reinterpret_cast<u32x2*>(out + col) = wh;
      *reinterpret_cast<u32x2*>(out + g.n + col) = wl;
    } else {   // EPI_STORE
      const int orow = g.out_rows ? g.out_rows[row] : row;
      uint16_t* out = reinterpret_cast<uint16_t*>(g.out) + (long)orow * g.ldc;
      u32x2 w;
      if (g.accumulate) {
        const u32x2 old = *reinterpret_cast<const u32x2*>(out + col);
        w[0] = pack2bf(lo_bf(old[0]) + bf2f(f2bf(a[0])), hi_bf(old[0]) + bf2f(f2bf(a[1])));
        w[1] = pack2bf(lo_bf(old[1]) + bf2f(f2bf(a[2])), hi_bf(old[1]) + bf2f(f2bf(a[3])));
      } else {
        w[0] = pack2bf(a[0], a[1]);
        w[1] = pack2bf(a[2], a[3]);
      }
      *reinterpret_cast<u32x2*>(out + col) = w;
    }
  }
}

template <int EPI, bool GATHER>
hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
  const int tiles_m = (g.m + BM - 1) / BM;
  constexpr bool kSwiglu = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SPLIT);
  const int tiles_n = kSwiglu ? (g.n / 2) / 128 : g.n / BN;
  const size_t lds = 2 * 2 * TILE_ELEMS * sizeof(uint16_t);
  // the dynamic-LDS limit is a per-device kernel attribute: set it once on
  // each device this instantiation is launched on (idempotent if two threads race)
  static std::atomic<unsigned long long> attr_devices{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = 1ull << (dev & 63);
  if (!(attr_devices.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tn_kernel<EPI, GATHER>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_devices.fetch_or(bit, std::memory_order_release);
  }
  const int ks = (EPI == EPI_PARTIAL) ? g.ksplit : 1;
  const int grid = ((tiles_m * tiles_n * ks + 7) / 8) * 8;     // a multiple of the 8 XCDs
  hipLaunchKernelGGL((gemm_tn_kernel<EPI, GATHER>), dim3(grid), dim3(NTHREADS), lds, s, g);
  return hipGetLastError();
}

// Cost model for the split count: workgroup waves over 256 CUs times the time
// of one 256x256 tile over its k range, plus the partial-sum round trip.
int choose_ksplit(int m, int k, int n) {
  const double tiles = (double)((m + BM - 1) / BM) * (n / BN);
  const double per_tile_s = 2.0 * BM * BN * (double)k / 4.4e12;     // ~1.1 PFLOP/s over 256 CUs
  int best = 1;
  double best_t = std::ceil(tiles / 256.0) * per_tile_s;
  for (int ks = 2; ks <= 16; ++ks) {
    if (k % (ks * BK) != 0) continue;
    const double t = std::ceil(tiles * ks / 256.0) * per_tile_s / ks + (double)ks * m * n * 8.0 / 5.0e12 + 4e-6;
    if (t < 0.9 * best_t) { best = ks; best_t = t; }
  }
  return best;
}

}  // namespace

int gemm_ksplit(int m, int k, int n, int epi) {
  if (epi != EPI_STORE && epi != EPI_ROPE && epi != EPI_SPLIT) return 1;
  return choose_ksplit(m, k, n);
}

size_t gemm_split_workspace(int m, int k, int n, int epi) {
  const int ks = gemm_ksplit(m, k, n, epi);
  return ks > 1 ? (size_t)ks * m * n * sizeof(float) : 0;
}

hipError_t launch_gemm(const GemmArgs& g0, int epi, hipStream_t s) {
  const bool gather = g0.a_rows != nullptr;
  GemmArgs g = g0;
  g.ksplit = 1;
  const int ks = gemm_ksplit(g.m, g.k, g.n, epi);
  if (ks > 1 && g.partial && g.partial_bytes >= (size_t)ks * g.m * g.n * sizeof(float)) {
    g.ksplit = ks;
    hipError_t e = gather ? launch_one<EPI_PARTIAL, true>(g, s) : launch_one<EPI_PARTIAL, false>(g, s);
    if (e != hipSuccess) return e;
    const long groups = (long)g.m * (g.n / 4);
    long blocks = (groups + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    switch (epi) {
      case EPI_STORE: hipLaunchKernelGGL(gemm_reduce_kernel<EPI_STORE>, dim3(blocks), dim3(256), 0, s, g); break;
      case EPI_ROPE: hipLaunchKernelGGL(gemm_reduce_kernel<EPI_ROPE>, dim3(blocks), dim3(256), 0, s, g); break;
      default: hipLaunchKernelGGL(gemm_reduce_kernel<EPI_SPLIT>, dim3(blocks), dim3(256), 0, s, g); break;
    }
    return hipGetLastError();
  }
  switch (epi) {
    case EPI_STORE: return gather ? launch_one<EPI_STORE, true>(g, s) : launch_one<EPI_STORE, false>(g, s);
    case EPI_ROPE: return gather ? launch_one<EPI_ROPE, true>(g, s) : launch_one<EPI_ROPE, false>(g, s);
    case EPI_SWIGLU: return gather ? launch_one<EPI_SWIGLU, true>(g, s) : launch_one<EPI_SWIGLU, false>(g, s);
    case EPI_KV: return gather ? launch_one<EPI_KV, true>(g, s) : launch_one<EPI_KV, false>(g, s);
    case EPI_SWIGLU_SPLIT: return launch_one<EPI_SWIGLU_SPLIT, false>(g, s);
    case EPI_SPLIT: return launch_one<EPI_SPLIT, false>(g, s);
    case EPI_SUMSQ: return launch_one<EPI_SUMSQ, false>(g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spts
