// bf16 "TN" GEMM on gfx950 MFMA: C[m, n] = A[m, k] * B[n, k]^T, fp32 accumulate.
//
// Used for every projection of an SPTS layer (K/V over all candidates, Q of
// the probe and selected rows, the O projection, the LTP proxy products and
// the reduced SwiGLU FFN).  Both operands are k-contiguous, so a wave reads
// each MFMA fragment as one 16-byte LDS load.
//
// Tiling: 256 x 256 x 64 per workgroup, 8 waves in a 4 (M) x 2 (N) grid, each
// wave owns a 64 x 128 block = 4 x 8 tiles of v_mfma_f32_16x16x32_bf16 (128
// fp32 accumulators per lane), two waves per SIMD.  On gfx950 the 16x16x32
// form kept the matrix cores busier than 32x32x16 with the same data flow.  Operands go straight from
// global memory into LDS, A and B each in two 32 KiB slots, copied by all 8
// waves.  Two barriers per k-step release the A slot and the B slot at
// different points, so the next steps' copies stay in flight across every
// barrier (see the pipeline comment in the kernel).
//
// The MFMA is issued as (B fragment, A fragment) so each lane's accumulators
// hold, per 16-row tile, ONE row of C and 4 consecutive columns of each
// 16-column tile; every epilogue (row scatter, RoPE pairs, SwiGLU pairs, row
// norms) is then lane-local.
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

// Epilogue of one finished 256 x 256 tile (STORE, ROPE, KV, SWIGLU,
// SWIGLU_SPLIT, SPLIT).  Lane holds C[row][col] for row = tile_m*BM + wm*64 +
// i*16 + r16 and col = (tile base) + wn*128 + j*16 + q4*4 + e (i < 4, j < 8,
// e < 4).  The wave's 128 columns are one RoPE head (column c pairs with
// c + 64: tile j with tile j + 4) or, for SwiGLU, 64 gate rows then the 64 up
// rows of the same outputs (again tile j with tile j + 4).
template <int EPI, bool GATHER>
__device__ __forceinline__ void store_tile(const GemmArgs& g, f32x4 (&acc)[4][8], int tile_m, int tile_n,
                                           bool part1, int wm, int wn, int r16, int q4) {
  constexpr bool kSwiglu = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SPLIT);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tile_m * BM + wm * 64 + i * 16 + r16;
    if (row >= g.m) continue;
    if (kSwiglu) {
      uint16_t* out = reinterpret_cast<uint16_t*>(g.out) + (long)row * g.ldc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gt = acc[i][j][e];
          const float up = acc[i][j + 4][e];
          hv[e] = (gt / (1.0f + __expf(-gt))) * up;
        }
        const int col = tile_n * 128 + wn * 64 + j * 16 + q4 * 4;
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
      for (int j = 0; j < 8; ++j) {
        float hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float t = acc[i][j][e];
          hi[e] = bf2f(f2bf(t));
          lo[e] = t - hi[e];
        }
        const int col = tile_n * BN + wn * 128 + j * 16 + q4 * 4;
        u32x2 wh, wl;
        wh[0] = pack2bf(hi[0], hi[1]); wh[1] = pack2bf(hi[2], hi[3]);
        wl[0] = pack2bf(lo[0], lo[1]); wl[1] = pack2bf(lo[2], lo[3]);
        *reinterpret_cast<u32x2*>(out + col) = wh;
        *reinterpret_cast<u32x2*>(out + g.n + col) = wl;
        if (g.split3) *reinterpret_cast<u32x2*>(out + 2 * g.n + col) = wh;
        if (g.tperm) *reinterpret_cast<f32x4*>(g.tperm + quad_perm(row, col, g.n)) = acc[i][j];
      }
      continue;
    }
    if (EPI == EPI_ROPE || (EPI == EPI_KV && !part1 && g.rope_table)) {
      const int arow = GATHER ? g.a_rows[row] : row;
      const float* tab = g.rope_table + (long)g.pos[arow] * 128;   // 64 (cos, sin) pairs
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = j * 16 + q4 * 4 + e;
          const float cs = tab[2 * c], sn = tab[2 * c + 1];
          const float x1 = acc[i][j][e], x2 = acc[i][j + 4][e];
          acc[i][j][e] = x1 * cs - x2 * sn;
          acc[i][j + 4][e] = x2 * cs + x1 * sn;
        }
    }
    // EPI_STORE / EPI_ROPE / EPI_KV
    const int orow = g.out_rows ? g.out_rows[row] : row;
    uint16_t* out = part1 ? reinterpret_cast<uint16_t*>(g.out2) + (long)orow * g.ldc2
                          : reinterpret_cast<uint16_t*>(g.out) + (long)orow * g.ldc;
    const int cshift = part1 ? g.n0 : 0;                  // KV: b1 columns restart at 0
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = tile_n * BN + wn * 128 + j * 16 + q4 * 4 - cshift;
      const f32x4 v = acc[i][j];
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

// Logical tile -> (tile_m, tile_n): the order walks groups of GROUP_M row
// tiles across all column tiles.
__device__ __forceinline__ void tile_of(int logical, int tiles_m, int tiles_n, int& tile_m, int& tile_n) {
  constexpr int GROUP_M = 4;
  const int in_group = GROUP_M * tiles_n;
  const int first_m = (logical / in_group) * GROUP_M;
  const int gm = min(GROUP_M, tiles_m - first_m);
  tile_m = first_m + (logical % in_group) % gm;
  tile_n = (logical % in_group) / gm;
}

// One fp32 tail piece of a tile, in the lanes' own register order: 32 groups
// of 16 bytes per thread (accumulator tile (i, j)), group-major, so each store
// covers 8 KiB contiguously.
__device__ __forceinline__ float* piece_base(const GemmArgs& g, int slot, int tid) {
  return g.partial + (size_t)slot * (BM * BN) + tid * 4;
}
__device__ __forceinline__ int piece_group(int i, int j) { return (i * 8 + j) * (NTHREADS * 4); }
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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
  const int r16 = lane & 15, q4 = lane >> 4;   // fragment row, 8-element k group

  // ---- work of this workgroup.  Workgroups are dealt round-robin to the 8
  // XCDs, so workgroup b runs on XCD b % 8.  Each XCD gets a contiguous run of
  // the logical tile order (see tile_of), so the ~32 tiles resident on one XCD
  // at a time form a 4 x 8 block that shares A and B k-slices in that XCD's L2.
  const int tiles_m = (g.m + BM - 1) / BM;
  constexpr bool kSwiglu = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SPLIT);
  constexpr bool kTail = (EPI == EPI_STORE || EPI == EPI_ROPE || EPI == EPI_KV || EPI == EPI_SWIGLU);
  const int tiles_n = kSwiglu ? (g.n / 2) / 128 : g.n / BN;
  const int ksplit = (EPI == EPI_PARTIAL || EPI == EPI_QUAD) ? g.ksplit : 1;
  const int b = (int)blockIdx.x;
  int logical, kslice = 0, k0, k1;
  int slot = -1, step = 0;             // tail piece slot; ends workgroups: tail tiles between jobs
  if (!kTail || g.tail_tiles == 0 || b < g.tail_full) {
    const int total = (kTail && g.tail_tiles) ? g.tail_full : tiles_m * tiles_n * ksplit;
    const int per_xcd = (total + 7) / 8;
    const int logical_k = (b & 7) * per_xcd + (b >> 3);
    if (logical_k >= total) return;                   // padding workgroups of the last XCD run
    kslice = logical_k % ksplit;                      // split-K slice (0 without split)
    logical = logical_k / ksplit;
    k0 = kslice * (g.k / BK / ksplit);
    k1 = k0 + g.k / BK / ksplit;
  } else {
    // tail units after the tail_full whole tiles (tail_full is a multiple of
    // 256, so b % 8 is still the XCD); units of one piece index (equal
    // pieces) or of one kind (heads, ends) run side by side at the same k.
    const int tb = b - g.tail_full;
    const int T = g.tail_tiles, KT = g.k / BK;
    const int E = g.tail_ends ? (T + g.tail_ends - 1) / g.tail_ends : 0;
    const int units = g.tail_ends ? T + E : T * g.tail_np;
    const int per_xcd = (units + 7) / 8;
    const int u = (tb & 7) * per_xcd + (tb >> 3);
    if (u >= units) return;
    int tt;
    if (g.tail_ends == 0) {
      const int piece = u / T;
      tt = u - piece * T;
      k0 = piece * KT / g.tail_np;
      k1 = (piece + 1) * KT / g.tail_np;
      slot = u;
    } else if (u < T) {
      tt = u; k0 = 0; k1 = g.tail_kx; slot = u;
    } else {
      tt = u - T; k0 = g.tail_kx; k1 = KT; slot = T + tt; step = E;
    }
    logical = g.tail_full + tt;
  }

  // one job = one tile over k-steps [k0, k1); only ends workgroups run more than one
  for (;;) {
    int tile_m, tile_n;
    tile_of(logical, tiles_m, tiles_n, tile_m, tile_n);

    // KV: tiles at or past column n0 read b1 and write out2
    const bool part1 = (EPI == EPI_KV) && tile_n * BN >= g.n0;

    // ---- direct global -> LDS staging by all 8 waves.  Wave w, instruction
    // i (0..3) of an operand writes the 1 KiB block of tile rows rb*8 ..
    // rb*8+7, rb = 8*i + w; lane L lands at row r = rb*8 + L/8, physical chunk
    // L%8, so it fetches the logical chunk (L%8) ^ ((r >> 1) & 7) -- the
    // swizzle of swz() applied on the global side.
    const int ld_sub = lane >> 3;                       // row within the 8-row block
    // byte offsets of the staged rows: A rows in 64 bits (a gathered source
    // can span more than 4 GiB), B rows in 32 bits (the host rejects weights
    // of 4 GiB or more)
    uint64_t a_off[4];
    uint32_t b_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rb = 8 * i + wave;
      const int r = rb * 8 + ld_sub;                    // row within the 256-row tile
      const int ld_ch = (lane & 7) ^ ((r >> 1) & 7);    // logical 16-byte chunk fetched
      int ar = tile_m * BM + r;
      if (ar >= g.m) ar = g.m - 1;
      if (GATHER) ar = g.a_rows[ar];
      a_off[i] = ((uint64_t)(uint32_t)ar * (uint32_t)g.lda + ld_ch * 8) * 2u;
      if (kSwiglu) {
        // wave column block r / 128: rows 0..63 gate, 64..127 up, same 64
        // outputs; block rb = 8*i + w covers rows 64..127 of its 128-row block
        // exactly when i is odd, so odd instructions read Wu
        const int within = r & 127;
        const uint32_t brow = (uint32_t)tile_n * 128 + (r >> 7) * 64 + (within & 63);
        b_off[i] = (brow * (uint32_t)g.ldb + ld_ch * 8) * 2u;
      } else {
        const uint32_t brow = (uint32_t)(tile_n * BN - (part1 ? g.n0 : 0)) + r;
        b_off[i] = (brow * (uint32_t)g.ldb + ld_ch * 8) * 2u;
      }
    }
    const char* abase = reinterpret_cast<const char*>(g.a);
    const char* b0base = reinterpret_cast<const char*>(part1 ? g.b1 : g.b0);
    const char* b1base = reinterpret_cast<const char*>(g.b1);
    const int KT = k1 - k0;                              // k-steps of this job
    const int kt_base = k0;
    // B's k offset wraps at kwrap when it is set; otherwise the modulus is
    // larger than any offset.  Kept free of a branch: a branch inside the
    // k-loop splits the last phase into two blocks and undoes its
    // MFMA / LDS-read interleave.
    const uint32_t kwr = g.kwrap > 0 ? (uint32_t)g.kwrap : 0x7fffffffu;

    // The operands of k-step s go to slots As[s & 1] and Bs[s & 1]; s past
    // the job's last step reloads that step (never read), so every wave
    // issues the same loads and addresses stay in bounds.
    auto issue_a = [&](int s) {
      const int kt = kt_base + (s < KT ? s : KT - 1);
      const uint32_t ka = (uint32_t)kt * BK * 2u;
      uint16_t* a_s = As + (s & 1) * TILE_ELEMS;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(abase + a_off[i] + ka),
            (__attribute__((address_space(3))) void*)(a_s + (8 * i + wave) * 512), 16, 0, 0);
    };
    auto issue_b = [&](int s) {
      const int kt = kt_base + (s < KT ? s : KT - 1);
      const uint32_t kb = ((uint32_t)(kt * BK) % kwr) * 2u;
      uint16_t* b_s = Bs + (s & 1) * TILE_ELEMS;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* bb = (kSwiglu && (i & 1)) ? b1base : b0base;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(bb + b_off[i] + kb),
            (__attribute__((address_space(3))) void*)(b_s + (8 * i + wave) * 512), 16, 0, 0);
      }
    };
    // fragments of 16 rows x 32 k (lane: row r16, elements 8*q4 .. 8*q4+7 of
    // the 32) for substep kk2 (k 32*kk2 .. 32*kk2+31 of the step)
    auto read_a = [&](bf16x8 (&f)[4], int s, int kk2) {
      const uint16_t* a_s = As + (s & 1) * TILE_ELEMS;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f[i] = *reinterpret_cast<const bf16x8*>(a_s + swz(wm * 64 + i * 16 + r16, kk2 * 4 + q4));
    };
    auto read_b = [&](bf16x8 (&f)[8], int s, int kk2) {
      const uint16_t* b_s = Bs + (s & 1) * TILE_ELEMS;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        f[j] = *reinterpret_cast<const bf16x8*>(b_s + swz(wn * 128 + j * 16 + r16, kk2 * 4 + q4));
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
    // the MFMAs of column tiles j0 .. j0+3
    auto mma = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[8], int j0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = j0; j < j0 + 4; ++j) acc[i][j] = mfma16x16x32(fb[j], fa[i], acc[i][j]);
    };

    // Pipeline.  A k-step is two 32-deep substeps, each issued as two phases
    // of 16 MFMAs (column tiles 0-3, then 4-7).  A step's A fragments are all
    // read by the end of its phase 1 and its B fragments by the end of phase
    // 0, so two barriers per step free the slots at different times: after
    // barrier M(t) (phase 1 done) the A slot of step t takes step t+2; after
    // barrier E(t) (phase 2 done, step t+1 landed) the B slot of step t takes
    // step t+2.  E waits only for step t+1's copies, so step t+2's A copies
    // stay in flight across it and the load pipeline never drains.
    bf16x8 fa0[4], fa1[4], fb0[8], fb1[8];
    issue_a(0);
    issue_b(0);
    issue_a(1);
    issue_b(1);
    __builtin_amdgcn_s_waitcnt(0x0070 | 8);   // vmcnt(8): step 0 landed, step 1 in flight
    __syncthreads();
    read_a(fa0, 0, 0);
    read_b(fb0, 0, 0);
    for (int kt = 0; kt < KT; ++kt) {
      // phase 0: substep 0, columns 0-3; B of substep 1
      read_b(fb1, kt, 1);
      mma(fa0, fb0, 0);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
      // phase 1: substep 0, columns 4-7; A of substep 1
      read_a(fa1, kt, 1);
      mma(fa0, fb0, 4);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
      __builtin_amdgcn_sched_barrier(0);
      // M(kt): every A read of step kt is done
      __builtin_amdgcn_s_waitcnt(0xC07F & ~0x0F00);   // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // phase 2: substep 1, columns 0-3; A of step kt+2 into the A slot of step kt
      issue_a(kt + 2);
      mma(fa1, fb1, 0);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // one copy
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
      __builtin_amdgcn_sched_barrier(0);
      // E(kt): every read of step kt is done; step kt+1 has landed (only the
      // four A copies of step kt+2 may still be in flight)
      __builtin_amdgcn_s_waitcnt(0x0070 | 4);   // vmcnt(4) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // phase 3: substep 1, columns 4-7; substep 0 of step kt+1; B of step
      // kt+2 into the B slot of step kt
      read_a(fa0, kt + 1, 0);
      read_b(fb0, kt + 1, 0);
      issue_b(kt + 2);
      mma(fa1, fb1, 4);
#pragma unroll
      for (int p = 0; p < 12; ++p) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // no copy into LDS outlives the k-loop, and no wave still reads it
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    if (kTail && slot >= 0) {
      float* ps = piece_base(g, slot, tid);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4*>(ps + piece_group(i, j)) = acc[i][j];
      if (step == 0) return;
      logical += step;
      slot += step;
      if (logical - g.tail_full >= g.tail_tiles) return;
      continue;
    }

    // ------------------------------------------------------------ epilogues
    // lane holds C[row][col] for row = tile_m*BM + wm*64 + i*16 + r16 and
    // col = (tile base) + wn*128 + j*16 + q4*4 + e.
    if (EPI == EPI_PARTIAL) {
      float* part = g.partial + (long)kslice * g.m * g.n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = tile_m * BM + wm * 64 + i * 16 + r16;
        if (row >= g.m) continue;
        float* prow = part + (long)row * g.n;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<f32x4*>(prow + tile_n * BN + wn * 128 + j * 16 + q4 * 4) = acc[i][j];
      }
      return;
    }
    if (EPI == EPI_QUAD) {
      // this k-slice's row sums of C[i, c] * t[i, c] over the tile's 256
      // columns, t in the lanes' own order (one coalesced 16-byte load per
      // accumulator tile; the padding rows past m are summed, never stored):
      // a lane's 32 columns, then the 4 lanes of the row (q4), then the two
      // column waves (LDS)
      float* red = reinterpret_cast<float*>(smem);   // [4 wm][4 i][16 rows] from wn == 1
      float ss[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = tile_m * BM + wm * 64 + i * 16 + r16;
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = tile_n * BN + wn * 128 + j * 16 + q4 * 4;
          const f32x4 tv = *reinterpret_cast<const f32x4*>(g.tperm + quad_perm(row, col, g.n));
          t += acc[i][j][0] * tv[0];
          t += acc[i][j][1] * tv[1];
          t += acc[i][j][2] * tv[2];
          t += acc[i][j][3] * tv[3];
        }
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        ss[i] = t;
      }
      if (wn == 1 && q4 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(wm * 4 + i) * 16 + r16] = ss[i];
      }
      __syncthreads();
      if (wn == 0 && q4 == 0) {
        float* out = reinterpret_cast<float*>(g.out);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = tile_m * BM + wm * 64 + i * 16 + r16;
          if (row < g.m)
            out[((long)row * tiles_n + tile_n) * ksplit + kslice] = ss[i] + red[(wm * 4 + i) * 16 + r16];
        }
      }
      return;
    }
    if (EPI == EPI_SUMSQ) {
      // row sums of squares over the tile's 256 columns: a lane's 32 columns,
      // then the 4 lanes of the row (q4), then the two column waves (LDS)
      float* red = reinterpret_cast<float*>(smem);   // [4 wm][4 i][16 rows] from wn == 1
      float ss[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) t += acc[i][j][e] * acc[i][j][e];
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        ss[i] = t;
      }
      if (wn == 1 && q4 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(wm * 4 + i) * 16 + r16] = ss[i];
      }
      __syncthreads();
      if (wn == 0 && q4 == 0) {
        float* out = reinterpret_cast<float*>(g.out);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = tile_m * BM + wm * 64 + i * 16 + r16;
          if (row < g.m) out[(long)row * tiles_n + tile_n] = ss[i] + red[(wm * 4 + i) * 16 + r16];
        }
      }
      return;
    }

    store_tile<EPI, GATHER>(g, acc, tile_m, tile_n, part1, wm, wn, r16, q4);
    return;
  }
}

// Tail fixup: tile tail_full + blockIdx.x is the fp32 sum of its tail_np
// pieces, added in k order, then finished by the GEMM's own epilogue.
template <int EPI, bool GATHER>
__global__ __launch_bounds__(NTHREADS) void gemm_tail_fixup_kernel(GemmArgs g) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, q4 = lane >> 4;   // fragment row, 8-element k group
  constexpr bool kSwiglu = (EPI == EPI_SWIGLU);
  const int tiles_m = (g.m + BM - 1) / BM;
  const int tiles_n = kSwiglu ? (g.n / 2) / 128 : g.n / BN;
  const int tt = (int)blockIdx.x;
  int tile_m, tile_n;
  tile_of(g.tail_full + tt, tiles_m, tiles_n, tile_m, tile_n);
  const bool part1 = (EPI == EPI_KV) && tile_n * BN >= g.n0;
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  for (int p = 0; p < g.tail_np; ++p) {
    const float* ps = piece_base(g, p * g.tail_tiles + tt, tid);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] += *reinterpret_cast<const f32x4*>(ps + piece_group(i, j));
  }
  store_tile<EPI, GATHER>(g, acc, tile_m, tile_n, part1, wm, wn, r16, q4);
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
      if (g.split3) *reinterpret_cast<u32x2*>(out + 2 * g.n + col) = wh;
      if (g.tperm) *reinterpret_cast<f32x4*>(g.tperm + quad_perm(row, col, g.n)) = a;
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
  const int ks = (EPI == EPI_PARTIAL || EPI == EPI_QUAD) ? g.ksplit : 1;
  int grid = ((tiles_m * tiles_n * ks + 7) / 8) * 8;           // a multiple of the 8 XCDs
  if (g.tail_tiles > 0) {
    const int units = g.tail_ends ? g.tail_tiles + (g.tail_tiles + g.tail_ends - 1) / g.tail_ends
                                  : g.tail_tiles * g.tail_np;
    grid = g.tail_full + ((units + 7) / 8) * 8;
  }
  hipLaunchKernelGGL((gemm_tn_kernel<EPI, GATHER>), dim3(grid), dim3(NTHREADS), lds, s, g);
  e = hipGetLastError();
  if constexpr (EPI == EPI_STORE || EPI == EPI_ROPE || EPI == EPI_KV || EPI == EPI_SWIGLU) {
    if (e == hipSuccess && g.tail_tiles > 0) {
      hipLaunchKernelGGL((gemm_tail_fixup_kernel<EPI, GATHER>), dim3(g.tail_tiles), dim3(NTHREADS), 0, s, g);
      e = hipGetLastError();
    }
  }
  return e;
}

// Cost model: workgroup rounds over 256 CUs times the time of one 256x256 tile
// over its k range, plus the round trip of any fp32 partial results.
//  - split-K (ksplit > 1): every tile in ksplit slices, summed by a reduce pass.
//  - tail split: the whole rounds run unsplit, and the tiles of the last,
//    partly filled round are cut along k so that they fill all 256 CUs.  With
//    at most 128 tail tiles each is cut into equal pieces, one workgroup per
//    piece; with more, each tile's head [0, kx) gets a workgroup and the other
//    workgroups take the ends [kx, KT) of `ends` tiles each, kx chosen so a
//    head and `ends` ends take equally long.  Workgroups that run side by
//    side then sit at the same k, as in the unsplit rounds, so they still
//    share operand k-slices in L2.  A second launch adds each tile's pieces.
constexpr int kCUs = 256;
constexpr double kTileFlops = 4.4e12;   // per-CU rate on one tile: ~1.1 PFLOP/s over 256 CUs
constexpr double kPartialBps = 4.5e12;  // fp32 partials written, then read back

struct Plan {
  int ksplit = 1;
  int full = 0, tiles = 0, np = 0, ends = 0, kx = 0;   // tail split when tiles > 0
  size_t ws = 0;                                       // fp32 workspace bytes
  double t = 0;                                        // modeled seconds
};

Plan choose_plan(int m, int k, int n, int epi) {
  const bool swiglu = (epi == EPI_SWIGLU || epi == EPI_SWIGLU_SPLIT);
  const int tiles = ((m + BM - 1) / BM) * (swiglu ? (n / 2) / 128 : n / BN);
  const int KT = k / BK;
  const double tile_s = 2.0 * BM * BN * (double)k / kTileFlops;
  Plan best;
  best.t = std::ceil(tiles / (double)kCUs) * tile_s;
  if (epi == EPI_STORE || epi == EPI_ROPE || epi == EPI_SPLIT) {
    for (int ks = 2; ks <= 16; ++ks) {
      if (k % (ks * BK) != 0) continue;
      const double t = std::ceil((double)tiles * ks / kCUs) * tile_s / ks + (double)ks * m * n * 8.0 / 5.0e12 + 4e-6;
      if (t < 0.9 * best.t) {
        best = Plan{};
        best.ksplit = ks; best.t = t; best.ws = (size_t)ks * m * n * sizeof(float);
      }
    }
  }
  const int T = tiles % kCUs;
  if ((epi == EPI_STORE || epi == EPI_ROPE || epi == EPI_KV || epi == EPI_SWIGLU) && T != 0 && KT >= 2) {
    Plan p;
    p.full = tiles - T;
    p.tiles = T;
    double steps;                        // k-steps of the longest tail workgroup
    if (2 * T <= kCUs) {
      p.np = std::min(kCUs / T, KT);
      steps = (KT + p.np - 1) / p.np;
    } else {
      p.np = 2;
      p.ends = (T + (kCUs - T) - 1) / (kCUs - T);
      p.kx = std::min(KT - 1, std::max(1, (int)std::lround((double)KT * p.ends / (p.ends + 1))));
      steps = std::max(p.kx, p.ends * (KT - p.kx));
    }
    p.ws = (size_t)T * p.np * BM * BN * sizeof(float);
    p.t = (p.full / kCUs + steps / KT) * tile_s + 2.0 * p.ws / kPartialBps + 6e-6 + p.ends * 2e-6;
    if (p.t < 0.97 * best.t) best = p;
  }
  return best;
}

}  // namespace

int gemm_ksplit(int m, int k, int n, int epi) { return choose_plan(m, k, n, epi).ksplit; }

// EPI_QUAD: the k-split (a divisor of the k-steps, at least two per slice)
// with the fewest rounds of workgroups times k-steps per slice, the smaller
// split on a tie.  The row sums are linear in C, so each slice finishes its
// own part and no fp32 tile goes through memory.
int gemm_quad_ksplit(int m, int k, int n) {
  const long tiles = (long)((m + BM - 1) / BM) * (n / BN);
  const int KT = k / BK;
  int best = 1;
  long best_cost = -1;
  for (int ks = 1; ks <= (KT >= 2 ? KT / 2 : 1); ++ks) {
    if (KT % ks != 0) continue;
    const long cost = ((tiles * ks + kCUs - 1) / kCUs) * (KT / ks);
    if (best_cost < 0 || cost < best_cost) {
      best = ks;
      best_cost = cost;
    }
  }
  return best;
}

size_t gemm_split_workspace(int m, int k, int n, int epi) { return choose_plan(m, k, n, epi).ws; }

hipError_t launch_gemm(const GemmArgs& g0, int epi, hipStream_t s) {
  const bool gather = g0.a_rows != nullptr;
  GemmArgs g = g0;
  g.ksplit = 1;
  g.tail_full = g.tail_tiles = g.tail_np = g.tail_ends = g.tail_kx = 0;
  const Plan plan = choose_plan(g.m, g.k, g.n, epi);
  const bool room = plan.ws > 0 && g.partial && g.partial_bytes >= plan.ws;
  if (room && plan.tiles > 0) {
    g.tail_full = plan.full; g.tail_tiles = plan.tiles; g.tail_np = plan.np;
    g.tail_ends = plan.ends; g.tail_kx = plan.kx;
  }
  if (epi == EPI_QUAD) {
    g.ksplit = gemm_quad_ksplit(g.m, g.k, g.n);
    return launch_one<EPI_QUAD, false>(g, s);
  }
  if (room && plan.ksplit > 1) {
    g.ksplit = plan.ksplit;
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
