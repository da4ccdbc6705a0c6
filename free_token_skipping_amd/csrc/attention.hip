// PAP probe scores and reduced (selected-query) causal attention, gfx950.
//
// Both use v_mfma_f32_32x32x16_bf16 with key/value tiles of 64 tokens staged
// in LDS and shared by the 4 waves of a workgroup; the 4 waves are 4 query
// heads of one GQA group, so each K/V tile is read from HBM once per group.
//
// Layout trick (reduced attention): logits are formed transposed,
// S^T = K Q^T, so a lane owns one query and the softmax statistics are
// lane-local.  The K rows fed to the MFMA are permuted (bits 2 and 3 of the
// row index swapped) so that the 16 logits a lane holds per 32-key tile are
// two runs of 8 CONSECUTIVE keys; those become, after exp and bf16
// rounding, the MFMA B operand of O^T = V^T P^T with no lane exchange, and
// the matching V^T fragment is a single 16-byte LDS read from a transposed
// V tile.
#include <type_traits>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace spts {
namespace {

constexpr int KT = 64;          // keys per LDS tile
constexpr int DH = 128;

// LDS swizzles.  gfx950 serves a 16-byte-per-lane LDS read 16 lanes at a
// time across 64 banks (256 bytes); the 16 rows read together must fall in
// 16 distinct 16-byte slots of that window.
// K tile [64 keys][128] (256-byte rows): chunk XOR (key & 15).
__device__ __forceinline__ int kswz(int key, int chunk) { return key * DH + ((chunk ^ (key & 15)) << 3); }
// V^T tile [128 dh][64 keys] (128-byte rows, two rows per window): chunk XOR ((dh >> 1) & 7).
__device__ __forceinline__ int vswz(int d, int chunk) { return d * KT + ((chunk ^ ((d >> 1) & 7)) << 3); }
// MFMA A-row -> key row within a 32-key tile: swap index bits 2 and 3.
__device__ __forceinline__ int perm32(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// Stage one K tile (and optionally the transposed V tile) of KV head g.
// Rows >= n are clamped to n-1 (they are always masked).
struct TileRegs { u32x4 k[4]; u32x4 v[4]; };

__device__ __forceinline__ void load_tile(TileRegs& t, const uint16_t* k, const uint16_t* v, int j0,
                                          int n, int Hkv, int g, int tid, bool with_v) {
  const long row_stride = (long)Hkv * DH;
#pragma unroll
  for (int i = 0; i < 4; ++i) {        // K: thread -> row tid/16 + 16 i, chunk tid%16
    int j = j0 + (tid >> 4) + 16 * i;
    j = j < n ? j : n - 1;
    t.k[i] = ld16(k + j * row_stride + g * DH + (tid & 15) * 8);
  }
  if (with_v) {                        // V: thread -> keys 4*(tid%16)+q, dh chunk tid/16
    const int kq4 = tid & 15, dc = tid >> 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int j = j0 + kq4 * 4 + q;
      j = j < n ? j : n - 1;
      t.v[q] = ld16(v + j * row_stride + g * DH + dc * 8);
    }
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& t, uint16_t* ks, uint16_t* vts, int tid,
                                           bool with_v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) st16(ks + kswz((tid >> 4) + 16 * i, tid & 15), t.k[i]);
  if (with_v) {
    const int kq4 = tid & 15, dc = tid >> 4;
    // transpose 4 keys x 8 dh -> 8 rows of 4 keys (8 bytes each)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      const bool hiw = e & 1;
      uint32_t x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = hiw ? (t.v[q][w] >> 16) : (t.v[q][w] & 0xFFFFu);
      u32x2 out;
      out[0] = x[0] | (x[1] << 16);
      out[1] = x[2] | (x[3] << 16);
      *reinterpret_cast<u32x2*>(vts + vswz(dc * 8 + e, kq4 >> 1) + (kq4 & 1) * 4) = out;
    }
  }
}

// ============================================================ reduced attention
// grid: ceil(kq/64) * Hq/4 workgroups, one per (64-query block, group of 4
// query heads); block 512 = 8 waves: wave w serves query head 4*hg + (w & 3)
// for the 32 queries q0 + 32*(w >> 2) .. +31 (two waves per SIMD).
//
// Software pipeline inside each wave, one 64-key tile per step: while the
// VALU turns the logits of tile t into bf16 probabilities, the MFMA unit forms
// the logits of tile t+1 and accumulates O += V_{t-1} P_{t-1} (the P of the
// previous step).  The three streams share no data, so they interleave one
// MFMA at a time; the exp2 stream hides almost entirely behind the matrix
// core.  Masking of tile t+1 and the reference-max update follow in the same
// step, after the overlapped block.
//
// The reference max is updated lazily: only when a lane's logits exceed it
// by more than 2^8 (exp2 units), so the O rescale is rare; p = exp2(s*scale*
// log2e - m) then stays <= 256 and O / l is exact whatever reference was used.
//
// LDS rows are padded by 16 bytes instead of XOR-swizzled: gfx950 serves a
// 16-byte-per-lane read 16 lanes at a time over a 256-byte bank window, and a
// row stride of 17 (K) or 9 (V^T) 16-byte slots puts the 16 rows read together
// in 16 distinct slots, while every fragment sits at a constant offset from
// one per-lane base address.
constexpr float kLazyMax = 8.0f;
constexpr int KROW = DH + 8;     // K tile row: 128 dh + 8 pad elements (272 B)
constexpr int VROW = KT + 8;     // V^T tile row: 64 keys + 8 pad elements (144 B)

__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(const uint16_t* __restrict__ q,
                                                           const int32_t* __restrict__ idx,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, int kq,
                                                           int n, int Hq, int Hkv, float sl2,
                                                           uint16_t* __restrict__ o) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][DH * VROW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  // Workgroup id -> (query block, 4-head group): all head groups of the
  // latest (longest) query block first, so the causal work shrinks
  // monotonically over the dispatch and the tail holds the short blocks.
  // Workgroup b runs on XCD b % 8, so with 8 head groups each XCD's L2 serves
  // one KV head.
  const int nqb = (kq + 63) >> 6;
  const int hgs = Hq >> 2;
  const int qb = nqb - 1 - (int)blockIdx.x / hgs;
  const int hg = (int)blockIdx.x % hgs;
  const int h = hg * 4 + (wave & 3);
  const int g = (hg * 4) / (Hq / Hkv);
  const int q0 = qb * 64;
  const int qw = q0 + (wave >> 2) * 32;              // this wave's first query

  const int qi_raw = qw + l32;
  const int qi = qi_raw < kq ? qi_raw : kq - 1;
  const int qpos = idx[qi];
  const int kmax = idx[min(q0 + 63, kq - 1)];
  const int ntiles = kmax / KT + 1;
  const int nfull = (idx[q0] + 1) / KT;             // tiles entirely below every query of the block

  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(q + ((long)qi * Hq + h) * DH + kk * 16 + half * 8);

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_ref = -INFINITY, l_part = 0.f;             // l_part: this half-wave's keys only
  const f32x16 zero16 = {};

  // per-lane LDS fragment bases (elements); fragments are at constant offsets
  const int kfrag = perm32(l32) * KROW + half * 8;   // + kt*32*KROW + kk*16
  const int vfrag = l32 * VROW + half * 8;           // + d*32*VROW + ks4*16

  // ---- staging: K rows (2 x 16 B / thread), V as 2-key x 8-dh blocks.
  // Element offsets fit in 32 bits (n * Hkv * 128 < 2^31 is checked on the host).
  const int row_stride = Hkv * DH;
  const uint16_t* kbase = k + g * DH + (tid & 15) * 8;
  const int kp = tid & 31, dc = tid >> 5;            // V: key pair, dh chunk
  const uint16_t* vbase = v + g * DH + dc * 8;
  u32x4 kr[2], vr[2];
  auto load_k = [&](int j0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = min(j0 + (tid >> 4) + 32 * i, n - 1);
      kr[i] = ld16(kbase + j * row_stride);
    }
  };
  auto load_v = [&](int j0) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = min(j0 + 2 * kp + e, n - 1);
      vr[e] = ld16(vbase + j * row_stride);
    }
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) st16(Ks[buf] + ((tid >> 4) + 32 * i) * KROW + (tid & 15) * 8, kr[i]);
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      const uint32_t a = (e & 1) ? (vr[0][w] >> 16) : (vr[0][w] & 0xFFFFu);
      const uint32_t b = (e & 1) ? (vr[1][w] >> 16) : (vr[1][w] & 0xFFFFu);
      *reinterpret_cast<uint32_t*>(Vs[buf] + (dc * 8 + e) * VROW + kp * 2) = a | (b << 16);
    }
  };
  // logits S^T = K_t Q^T (64 keys, rows permuted, x 32 queries)
  auto logits = [&](int buf, f32x16 (&sd)[2]) {
    const uint16_t* ks = Ks[buf] + kfrag;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + kt * 32 * KROW + kk * 16);
        sd[kt] = mfma32x32x16(kf, qf[kk], kk == 0 ? zero16 : sd[kt]);
      }
  };
  // mask tile t's keys beyond each query, then move the reference max if
  // needed; key of reg r = t*64 + kt*32 + (r>>3)*16 + half*8 + (r&7).  `pend`
  // is the P of the previous tile, already formed against the old reference
  // but not yet multiplied into O: a move rescales it together with O and l.
  auto prepare = [&](int t, f32x16 (&sd)[2], bf16x8 (&pend)[4]) {
    if (t >= nfull) {
      const int j0 = t * KT;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kt * 32 + (r >> 3) * 16 + half * 8 + (r & 7);
          if (key > qpos) sd[kt][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sd[kt][r]), sd[kt][r + 1]);
    mx *= sl2;
    if (__any(mx > m_ref + kLazyMax)) {
      const float m_new = fmaxf(m_ref, fmaxf(mx, __shfl_xor(mx, 32)));
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f32x8 pv = __builtin_convertvector(pend[c], f32x8);
        pv *= alpha;
        pend[c] = __builtin_convertvector(pv, bf16x8);
      }
      m_ref = m_new;
    }
  };
  // P_t = exp2(logit * scale * log2e - m_ref) as bf16 MFMA operands; l += P_t
  auto softmax = [&](f32x16 (&sc)[2], bf16x8 (&pc)[4]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kt][sub * 8 + e], sl2, -m_ref));
          l_part += pv[e];
        }
        pc[kt * 2 + sub] = __builtin_convertvector(pv, bf16x8);
      }
  };
  // O^T += V_u^T P_u^T, V_u in buffer vb
  auto pv_mma = [&](int vb, bf16x8 (&pp)[4]) {
    const uint16_t* vs = Vs[vb] + vfrag;
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs + d * 32 * VROW + ks4 * 16);
        oacc[d] = mfma32x32x16(vf, pp[ks4], oacc[d]);
      }
  };

  // One pipeline step t.  sc holds tile t's logits (masked, reference max
  // set), pp the P of tile t-1.  The matrix core forms the logits of tile t+1
  // and O += P_{t-1} V_{t-1} while the VALU turns tile t's logits into P_t, so
  // all three streams are independent and interleave one MFMA at a time.  V
  // trails K by two tiles: V_t is staged during step t (into buffer t & 1)
  // and read at step t+1, K_{t+2} is staged during step t.
  auto step = [&](auto with_pv, int t, f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pp)[4],
                  bf16x8 (&pc)[4]) {
    constexpr bool kPV = decltype(with_pv)::value;
    // K/V staging is unconditional (rows clamp to n-1; past the last tile the
    // K store lands in buffer t & 1, whose tile was read in step t-1), so no
    // branch splits the MFMA / VALU block
    load_k((t + 2) * KT);
    load_v(t * KT);
    logits((t + 1) & 1, sn);             // stale data past the last tile; unused
    if constexpr (kPV) pv_mma((t - 1) & 1, pp);
    softmax(sc, pc);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);          // first K fragments
    if constexpr (kPV) {
#pragma unroll
      for (int r = 0; r < 28; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // next K / V fragment
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);      // softmax VALU + exp
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 12; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);
      }
    }
    // P_t is only read in the next step; without this anchor the compiler
    // sinks the softmax below the masking of tile t+1, away from the MFMAs
    asm volatile("" : "+v"(pc[0]), "+v"(pc[1]), "+v"(pc[2]), "+v"(pc[3]), "+v"(l_part));
    store_k(t & 1);
    store_v(t & 1);
    if (t + 1 < ntiles) prepare(t + 1, sn, pc);
    __syncthreads();
  };

  // prologue: K_0, K_1 staged; logits of tile 0
  load_k(0);
  store_k(0);
  if (ntiles > 1) {
    load_k(KT);
    store_k(1);
  }
  __syncthreads();
  f32x16 sa[2], sb[2];
  bf16x8 pa[4], pb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    pa[c] = bf16x8{};
    pb[c] = bf16x8{};
  }
  logits(0, sa);
  prepare(0, sa, pb);                     // nothing pending yet (pb is zero)
  step(std::false_type{}, 0, sa, sb, pb, pa);
  int t = 1;
  for (; t + 1 < ntiles; t += 2) {
    step(std::true_type{}, t, sb, sa, pa, pb);
    step(std::true_type{}, t + 1, sa, sb, pb, pa);
  }
  if (t < ntiles) step(std::true_type{}, t, sb, sa, pa, pb);
  // the last tile's P: step t leaves P_t in pb for odd t, in pa for even t
  if ((ntiles - 1) & 1) pv_mma((ntiles - 1) & 1, pb);
  else pv_mma((ntiles - 1) & 1, pa);

  // normalise and store: lane = query, reg r of dh tile d -> dh d*32 + (r>>2)*8 + half*4 + (r&3)
  if (qi_raw < kq) {
    const float inv = 1.0f / (l_part + __shfl_xor(l_part, 32));
    uint16_t* orow = o + ((long)qi * Hq + h) * DH;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        u32x2 w;
        w[0] = pack2bf(oacc[d][qd * 4 + 0] * inv, oacc[d][qd * 4 + 1] * inv);
        w[1] = pack2bf(oacc[d][qd * 4 + 2] * inv, oacc[d][qd * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d * 32 + qd * 8 + half * 4) = w;
      }
  }
}

// =============================================================== PAP probe
// Pass 1: per key chunk, per head, partial (max, sum) of the probe softmax
// in log2 units.  grid (ceil(n/chunk), Hq/4), 4 waves = 4 heads.  A chunk is
// a multiple of the 64-key tile between 128 and 1024 keys: the shortest whose
// grid still fits in one round of resident workgroups (two per compute unit
// for P <= 64, one for P = 128, as the kernels' registers allow).  A partly
// filled second round costs a whole chunk's time, while every workgroup also
// loads all P probe queries of its 4 heads, so chunks stay as long as that
// round allows; past 1024 keys the grid runs in several rounds.
constexpr int MIN_CHUNK = 128;

int probe_chunk(int n, int Hq, int P) {
  const long slots = 256L * (P <= 64 ? 2 : 1);
  const long need = ((long)n * (Hq / 4) + slots - 1) / slots;      // keys per chunk for one round
  const int c = (int)(((need + KT - 1) / KT) * KT);
  return c < MIN_CHUNK ? MIN_CHUNK : (c > 1024 ? 1024 : c);
}

template <int PT>   // probe column tiles of 32 (P = 32*PT)
__global__ __launch_bounds__(256, 1) void probe_stats_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k, int n,
                                                             int chunk_keys,
                                                             int Hq, int Hkv, float sl2,
                                                             float* __restrict__ part_m,
                                                             float* __restrict__ part_l) {
  constexpr int P = 32 * PT;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * DH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int h = blockIdx.y * 4 + wave;
  const int g = (blockIdx.y * 4) / (Hq / Hkv);
  const int chunk = blockIdx.x;
  const int nt = min(chunk_keys / KT, (n - chunk * chunk_keys + KT - 1) / KT);   // key tiles of this chunk

  // tile t is read from Ks[t & 1] while tile t+1 is in flight in registers
  TileRegs tr;
  load_tile(tr, k, nullptr, chunk * chunk_keys, n, Hkv, g, tid, false);
  bf16x8 qf[PT][8];
#pragma unroll
  for (int c = 0; c < PT; ++c)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[c][kk] = *reinterpret_cast<const bf16x8*>(q + ((long)(c * 32 + l32) * Hq + h) * DH + kk * 16 + half * 8);
  float m[PT], l[PT];
#pragma unroll
  for (int c = 0; c < PT; ++c) { m[c] = -INFINITY; l[c] = 0.f; }
  store_tile(tr, Ks[0], nullptr, tid, false);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int j0 = chunk * chunk_keys + t * KT;
    if (t + 1 < nt) load_tile(tr, k, nullptr, j0 + KT, n, Hkv, g, tid, false);
    const uint16_t* kt_s = Ks[t & 1];
#pragma unroll
    for (int c = 0; c < PT; ++c) {
      const int prow = n - P + c * 32 + l32;
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt_s + kswz(kt * 32 + perm32(l32), kk * 2 + half));
          s[kt] = mfma32x32x16(kf, qf[c][kk], s[kt]);
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kt * 32 + (r >> 3) * 16 + half * 8 + (r & 7);
          float x = s[kt][r] * sl2;
          if (key > prow) x = -INFINITY;
          s[kt][r] = x;
          mx = fmaxf(mx, x);
        }
      const float mnew = fmaxf(m[c], mx);
      if (mnew == -INFINITY) continue;     // nothing visible yet for this probe
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) rs += __builtin_amdgcn_exp2f(s[kt][r] - mnew);
      l[c] = l[c] * __builtin_amdgcn_exp2f(m[c] - mnew) + rs;
      m[c] = mnew;
    }
    // the next tile goes to the other buffer, read last in step t-1 (before
    // the barrier that ended it)
    if (t + 1 < nt) store_tile(tr, Ks[(t + 1) & 1], nullptr, tid, false);
    __syncthreads();
  }
  // merge the two half-waves (they hold different keys of the same probes)
#pragma unroll
  for (int c = 0; c < PT; ++c) {
    const float m2 = __shfl_xor(m[c], 32), l2 = __shfl_xor(l[c], 32);
    const float mt = fmaxf(m[c], m2);
    float lt = 0.f;
    if (mt != -INFINITY) lt = l[c] * exp2f(m[c] - mt) + l2 * exp2f(m2 - mt);
    if (half == 0) {
      const long o = ((long)chunk * Hq + h) * P + c * 32 + l32;
      part_m[o] = mt;
      part_l[o] = lt;
    }
  }
}

// Pass 1b: combine chunk partials -> per (head, probe) max and 1/sum.  One
// wave per (head, probe); lanes stride over chunks, fixed-order wave tree.
__global__ __launch_bounds__(256) void probe_combine_kernel(const float* __restrict__ part_m,
                                                            const float* __restrict__ part_l, int nchunks,
                                                            int HP, float* __restrict__ fin_m,
                                                            float* __restrict__ fin_il) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= HP) return;
  float mt = -INFINITY;
  for (int c = lane; c < nchunks; c += 64) mt = fmaxf(mt, part_m[(long)c * HP + i]);
  mt = wave_max(mt);
  float lt = 0.f;
  for (int c = lane; c < nchunks; c += 64) {
    const float mc = part_m[(long)c * HP + i];
    if (mc != -INFINITY) lt += part_l[(long)c * HP + i] * exp2f(mc - mt);
  }
  lt = wave_sum(lt);
  if (lane == 0) {
    fin_m[i] = mt;
    fin_il[i] = 1.0f / lt;
  }
}

// Pass 2: column sums of the normalised probe softmax for one key chunk and
// one head quad; logits formed as S = Q K^T so a lane owns one key.
template <int PT>
__global__ __launch_bounds__(256, 1) void probe_colsum_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k, int n,
                                                              int chunk_keys,
                                                              int Hq, int Hkv, float sl2,
                                                              const float* __restrict__ fin_m,
                                                              const float* __restrict__ fin_il,
                                                              float* __restrict__ quad_sum) {
  constexpr int P = 32 * PT;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * DH];
  __shared__ __attribute__((aligned(16))) float st_m[4][P];
  __shared__ __attribute__((aligned(16))) float st_il[4][P];
  __shared__ float red[2][4][KT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int h = blockIdx.y * 4 + wave;
  const int g = (blockIdx.y * 4) / (Hq / Hkv);
  const int chunk = blockIdx.x;
  const int nt = min(chunk_keys / KT, (n - chunk * chunk_keys + KT - 1) / KT);   // key tiles of this chunk

  // tile t is read from Ks[t & 1] while tile t+1 is in flight in registers
  TileRegs tr;
  load_tile(tr, k, nullptr, chunk * chunk_keys, n, Hkv, g, tid, false);
  for (int i = tid; i < 4 * P; i += 256) {
    const int hh = blockIdx.y * 4 + i / P, p = i % P;
    st_m[i / P][p] = fin_m[hh * P + p];
    st_il[i / P][p] = fin_il[hh * P + p];
  }
  bf16x8 qf[PT][8];
#pragma unroll
  for (int c = 0; c < PT; ++c)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[c][kk] = *reinterpret_cast<const bf16x8*>(q + ((long)(c * 32 + l32) * Hq + h) * DH + kk * 16 + half * 8);

  store_tile(tr, Ks[0], nullptr, tid, false);
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int j0 = chunk * chunk_keys + t * KT;
    if (t + 1 < nt) load_tile(tr, k, nullptr, j0 + KT, n, Hkv, g, tid, false);
    const uint16_t* kt_s = Ks[t & 1];
    float colsum[2] = {0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = j0 + kt * 32 + perm32(l32);          // this lane's key column
      bf16x8 kf[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8*>(kt_s + kswz(kt * 32 + perm32(l32), kk * 2 + half));
#pragma unroll
      for (int c = 0; c < PT; ++c) {
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) s = mfma32x32x16(qf[c][kk], kf[kk], s);
        // reg r -> probe row p = c*32 + (r>>2)*8 + half*4 + (r&3)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int pb = c * 32 + qd * 8 + half * 4;
          const f32x4 mm = *reinterpret_cast<const f32x4*>(&st_m[wave][pb]);
          const f32x4 il = *reinterpret_cast<const f32x4*>(&st_il[wave][pb]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int prow = n - P + pb + e;
            if (key <= prow) colsum[kt] += __builtin_amdgcn_exp2f(s[qd * 4 + e] * sl2 - mm[e]) * il[e];
          }
        }
      }
    }
    // add the other half-wave (other probe rows), then the 4 heads
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) colsum[kt] += __shfl_xor(colsum[kt], 32);
    float(*rd)[KT] = red[t & 1];
    if (half == 0) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) rd[wave][kt * 32 + perm32(l32)] = colsum[kt];
    }
    if (t + 1 < nt) store_tile(tr, Ks[(t + 1) & 1], nullptr, tid, false);
    __syncthreads();
    if (tid < KT && j0 + tid < n)
      quad_sum[(long)blockIdx.y * n + j0 + tid] = ((rd[0][tid] + rd[1][tid]) + rd[2][tid]) + rd[3][tid];
  }
}

// Final: S[j] = sum over head quads, fixed order.
__global__ void quad_reduce_kernel(const float* __restrict__ quad_sum, int nq, int n, float* __restrict__ s) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  float t = 0.f;
  for (int i = 0; i < nq; ++i) t += quad_sum[(long)i * n + j];
  s[j] = t;
}

// ================================================== fp32 paths (small cases)
// One thread per (head, probe): causal row max and sum.
__global__ void probe_stats_f32_kernel(const float* q, const float* k, int n, int P, int Hq, int Hkv,
                                       int dh, float scale, float* fin_m, float* fin_il) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Hq * P) return;
  const int h = i / P, p = i % P, g = h / (Hq / Hkv), row = n - P + p;
  const float* qr = q + ((long)p * Hq + h) * dh;
  float mx = -INFINITY, sum = 0.f;
  for (int j = 0; j <= row; ++j) {
    const float* kr = k + ((long)j * Hkv + g) * dh;
    float dot = 0.f;
    for (int e = 0; e < dh; ++e) dot += qr[e] * kr[e];
    const float x = dot * scale;
    if (x > mx) { sum = sum * expf(mx - x) + 1.f; mx = x; } else { sum += expf(x - mx); }
  }
  fin_m[h * P + p] = mx;
  fin_il[h * P + p] = 1.f / sum;
}

__global__ void probe_colsum_f32_kernel(const float* q, const float* k, int n, int P, int Hq, int Hkv,
                                        int dh, float scale, const float* fin_m, const float* fin_il,
                                        float* s) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  float tot = 0.f;
  for (int h = 0; h < Hq; ++h) {
    const int g = h / (Hq / Hkv);
    const float* kr = k + ((long)j * Hkv + g) * dh;
    for (int p = 0; p < P; ++p) {
      if (j > n - P + p) continue;
      const float* qr = q + ((long)p * Hq + h) * dh;
      float dot = 0.f;
      for (int e = 0; e < dh; ++e) dot += qr[e] * kr[e];
      tot += expf(dot * scale - fin_m[h * P + p]) * fin_il[h * P + p];
    }
  }
  s[j] = tot;
}

// One 64-lane block per (query, head); lane e owns dh elements e and e+64.
__global__ void attn_f32_kernel(const float* q, const int32_t* idx, const float* k, const float* v,
                                int kq, int n, int Hq, int Hkv, int dh, float scale, float* o) {
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int g = h / (Hq / Hkv), row = idx[i];
  const float* qr = q + ((long)i * Hq + h) * dh;
  const float q0 = lane < dh ? qr[lane] : 0.f;
  const float q1 = lane + 64 < dh ? qr[lane + 64] : 0.f;
  float mx = -INFINITY, sum = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j = 0; j <= row; ++j) {
    const float* kr = k + ((long)j * Hkv + g) * dh;
    const float* vr = v + ((long)j * Hkv + g) * dh;
    float part = (lane < dh ? q0 * kr[lane] : 0.f) + (lane + 64 < dh ? q1 * kr[lane + 64] : 0.f);
    const float x = wave_sum(part) * scale;
    const float mnew = fmaxf(mx, x);
    const float a = expf(mx - mnew), p = expf(x - mnew);
    sum = sum * a + p;
    o0 = o0 * a + (lane < dh ? p * vr[lane] : 0.f);
    o1 = o1 * a + (lane + 64 < dh ? p * vr[lane + 64] : 0.f);
    mx = mnew;
  }
  float* orow = o + ((long)i * Hq + h) * dh;
  if (lane < dh) orow[lane] = o0 / sum;
  if (lane + 64 < dh) orow[lane + 64] = o1 / sum;
}

}  // namespace

// ---------------------------------------------------------------- launchers
size_t probe_workspace(int n, int P, int Hq) {
  const size_t nchunks = (size_t)(n + MIN_CHUNK - 1) / MIN_CHUNK;   // bound for every chunk size
  const size_t HP = (size_t)Hq * P;
  // part_m, part_l [nchunks*HP]; fin_m, fin_il [HP]; quad_sum [Hq/4 * n]
  size_t b = 2 * nchunks * HP * 4 + 2 * HP * 4 + (size_t)((Hq + 3) / 4) * n * 4;
  return (b + 255) & ~(size_t)255;
}

hipError_t launch_probe_bf16(const uint16_t* q, const uint16_t* k, int n, int P, int Hq, int Hkv,
                             float scale, float* scores, void* ws, hipStream_t s) {
  const int ck = probe_chunk(n, Hq, P);
  const int nchunks = (n + ck - 1) / ck;
  const long HP = (long)Hq * P;
  float* part_m = reinterpret_cast<float*>(ws);
  float* part_l = part_m + nchunks * HP;
  float* fin_m = part_l + nchunks * HP;
  float* fin_il = fin_m + HP;
  float* quad = fin_il + HP;
  const float sl2 = scale * kLog2e;
  const dim3 grid(nchunks, Hq / 4);
  switch (P / 32) {
#define SPTS_PROBE_CASE(PT)                                                                        \
  case PT:                                                                                         \
    hipLaunchKernelGGL(probe_stats_kernel<PT>, grid, dim3(256), 0, s, q, k, n, ck, Hq, Hkv, sl2,  \
                       part_m, part_l);                                                            \
    hipLaunchKernelGGL(probe_combine_kernel, dim3((HP + 3) / 4), dim3(256), 0, s, part_m,         \
                       part_l, nchunks, (int)HP, fin_m, fin_il);                                   \
    hipLaunchKernelGGL(probe_colsum_kernel<PT>, grid, dim3(256), 0, s, q, k, n, ck, Hq, Hkv, sl2, \
                       fin_m, fin_il, quad);                                                       \
    break;
    SPTS_PROBE_CASE(1)
    SPTS_PROBE_CASE(2)
    SPTS_PROBE_CASE(4)
#undef SPTS_PROBE_CASE
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(quad_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, quad, Hq / 4, n, scores);
  return hipGetLastError();
}

hipError_t launch_probe_f32(const float* q, const float* k, int n, int P, int Hq, int Hkv, int dh,
                            float scale, float* scores, void* ws, hipStream_t s) {
  float* fin_m = reinterpret_cast<float*>(ws);
  float* fin_il = fin_m + Hq * P;
  hipLaunchKernelGGL(probe_stats_f32_kernel, dim3((Hq * P + 127) / 128), dim3(128), 0, s, q, k, n, P,
                     Hq, Hkv, dh, scale, fin_m, fin_il);
  hipLaunchKernelGGL(probe_colsum_f32_kernel, dim3((n + 127) / 128), dim3(128), 0, s, q, k, n, P, Hq,
                     Hkv, dh, scale, fin_m, fin_il, scores);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const uint16_t* q, const int32_t* idx, const uint16_t* k,
                            const uint16_t* v, int kq, int n, int Hq, int Hkv, float scale,
                            uint16_t* o, hipStream_t s) {
  const dim3 grid(((kq + 63) / 64) * (Hq / 4));
  hipLaunchKernelGGL(attn_bf16_kernel, grid, dim3(512), 0, s, q, idx, k, v, kq, n, Hq, Hkv,
                     scale * kLog2e, o);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const float* q, const int32_t* idx, const float* k, const float* v,
                           int kq, int n, int Hq, int Hkv, int dh, float scale, float* o,
                           hipStream_t s) {
  hipLaunchKernelGGL(attn_f32_kernel, dim3(kq, Hq), dim3(64), 0, s, q, idx, k, v, kq, n, Hq, Hkv, dh,
                     scale, o);
  return hipGetLastError();
}

}  // namespace spts
