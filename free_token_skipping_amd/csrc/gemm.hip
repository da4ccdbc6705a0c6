// bf16 "TN" GEMM on gfx950 MFMA: C[m, n] = A[m, k] * B[n, k]^T, fp32 accumulate.
//
// Used for every projection of an SPTS layer (K/V over all candidates, Q of
// the probe and selected rows, the O projection, the LTP proxy products and
// the reduced SwiGLU FFN).  Both operands are k-contiguous, so a wave reads
// each MFMA fragment as one 16-byte LDS load.
//
// Tiling: 256 x 256 x 64 per workgroup, 4 waves in a 2 x 2 grid, each wave
// owns a 128 x 128 block = 4 x 4 tiles of v_mfma_f32_32x32x16_bf16 (256 fp32
// accumulators per lane).  Global -> registers -> LDS staging, double-buffered
// LDS (2 x 64 KiB), one barrier per k-step.  LDS rows are 128 B with the
// 16-byte chunk index XOR-ed with (row & 7), so the 8 lanes that share a bank
// window always hit 8 distinct chunks.
//
// The MFMA is issued as (B fragment, A fragment) so each lane's accumulators
// hold ONE row of C and 4 groups of 4 consecutive columns; every epilogue
// (row scatter, RoPE pairs, SwiGLU pairs, row norms) is then lane-local.
#include "common.hpp"
#include "kernels.hpp"

namespace spts {
namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 256;
constexpr int TILE_ELEMS = BM * BK;  // per operand per stage

__device__ __forceinline__ int swz(int row, int chunk) {  // element offset in a 64-wide LDS tile
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

template <int EPI, bool GATHER>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_tn_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* As = smem;                       // [2][BM*BK]
  uint16_t* Bs = smem + 2 * TILE_ELEMS;      // [2][BN*BK]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, half = lane >> 5;

  const int tiles_m = (g.m + BM - 1) / BM;
  const int tile_m = blockIdx.x % tiles_m;
  const int tile_n = blockIdx.x / tiles_m;

  // ---- per-thread global source offsets for the 8 A rows and 8 B rows it stages
  const int ld_row = tid >> 3;   // + 32 * i
  const int ld_ch = tid & 7;
  long a_off[8], b_off[8];
  unsigned b_from_up = 0;   // SWIGLU: bit i set when staged B row i comes from the up weight
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = tile_m * BM + ld_row + 32 * i;
    if (r >= g.m) r = g.m - 1;
    if (GATHER) r = g.a_rows[r];
    a_off[i] = (long)r * g.lda + ld_ch * 8;
    const int br = ld_row + 32 * i;
    if (EPI == EPI_SWIGLU) {
      // wave column block wn = br / 128: rows 0..63 gate, 64..127 up, same 64 outputs
      const int bw = br >> 7, within = br & 127;
      const long brow = (long)tile_n * 128 + bw * 64 + (within & 63);
      if (within >= 64) b_from_up |= 1u << i;
      b_off[i] = brow * g.ldb + ld_ch * 8;
    } else {
      b_off[i] = ((long)tile_n * BN + br) * g.ldb + ld_ch * 8;
    }
  }

  u32x4 ra[8], rb[8];
  const int KT = g.k / BK;

  auto load_global = [&](int kt) {
    const long ka = (long)kt * BK;
    const long kb = g.kwrap > 0 ? (ka % g.kwrap) : ka;
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = ld16(g.a + a_off[i] + ka);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (EPI == EPI_SWIGLU) {
        const uint16_t* base = ((b_from_up >> i) & 1u) ? g.b1 : g.b0;
        rb[i] = ld16(base + b_off[i] + kb);
      } else {
        rb[i] = ld16(g.b0 + b_off[i] + kb);
      }
    }
  };
  auto store_lds = [&](int buf) {
    uint16_t* a_s = As + buf * TILE_ELEMS;
    uint16_t* b_s = Bs + buf * TILE_ELEMS;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = ld_row + 32 * i;
      st16(a_s + swz(r, ld_ch), ra[i]);
      st16(b_s + swz(r, ld_ch), rb[i]);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_global(kt + 1);
    const uint16_t* a_s = As + cur * TILE_ELEMS;
    const uint16_t* b_s = Bs + cur * TILE_ELEMS;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[4], bfm[4];
      const int ch = kk * 2 + half;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(a_s + swz(wm * 128 + i * 32 + l32, ch));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfm[j] = *reinterpret_cast<const bf16x8*>(b_s + swz(wn * 128 + j * 32 + l32, ch));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(bfm[j], af[i], acc[i][j]);
    }
    if (kt + 1 < KT) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogues
  // lane holds C[row][col] for row = tile_m*BM + wm*128 + i*32 + l32 and
  // col = (tile base) + wn*128 + j*32 + q*8 + half*4 + e, r = q*4 + e.
  if (EPI == EPI_SUMSQ) {
    float* red = reinterpret_cast<float*>(smem);   // [2 wm][4 i][32 rows] from wn == 1
    float ss[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
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
      for (int i = 0; i < 4; ++i) red[(wm * 4 + i) * 32 + l32] = ss[i];
    }
    __syncthreads();
    if (wn == 0 && half == 0) {
      float* out = reinterpret_cast<float*>(g.out);
      const int tiles_n = g.n / BN;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = tile_m * BM + wm * 128 + i * 32 + l32;
        if (row < g.m) out[(long)row * tiles_n + tile_n] = ss[i] + red[(wm * 4 + i) * 32 + l32];
      }
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tile_m * BM + wm * 128 + i * 32 + l32;
    if (row >= g.m) continue;
    if (EPI == EPI_SWIGLU) {
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
    if (EPI == EPI_ROPE) {
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
    // EPI_STORE / EPI_ROPE
    const int orow = g.out_rows ? g.out_rows[row] : row;
    uint16_t* out = reinterpret_cast<uint16_t*>(g.out) + (long)orow * g.ldc;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = tile_n * BN + wn * 128 + j * 32 + q * 8 + half * 4;
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

template <int EPI, bool GATHER>
hipError_t launch_one(const GemmArgs& g, hipStream_t s) {
  const int tiles_m = (g.m + BM - 1) / BM;
  const int tiles_n = (EPI == EPI_SWIGLU) ? (g.n / 2) / 128 : g.n / BN;
  const size_t lds = 2 * 2 * TILE_ELEMS * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tn_kernel<EPI, GATHER>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_tn_kernel<EPI, GATHER>), dim3(tiles_m * tiles_n), dim3(NTHREADS), lds, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, int epi, hipStream_t s) {
  const bool gather = g.a_rows != nullptr;
  switch (epi) {
    case EPI_STORE: return gather ? launch_one<EPI_STORE, true>(g, s) : launch_one<EPI_STORE, false>(g, s);
    case EPI_ROPE: return gather ? launch_one<EPI_ROPE, true>(g, s) : launch_one<EPI_ROPE, false>(g, s);
    case EPI_SWIGLU: return gather ? launch_one<EPI_SWIGLU, true>(g, s) : launch_one<EPI_SWIGLU, false>(g, s);
    case EPI_SPLIT: return launch_one<EPI_SPLIT, false>(g, s);
    case EPI_SUMSQ: return launch_one<EPI_SUMSQ, false>(g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spts
