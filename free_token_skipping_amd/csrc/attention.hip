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
// core.  The check of tile t's weights and the masking of tile t+1 follow
// in the same step, after the overlapped block.
//
// No running max is taken per logit: p = exp2(s*scale*log2e - m) is formed
// against the current reference m, and only when a lane's 32 weights of a
// tile sum to more than 2^64 (or to inf or NaN) is the tile redone against
// the exact max, which becomes the reference (a rare O rescale).  The first
// tile's exact max sets the initial reference.  Every p then stays <= 2^64
// (a bf16 holds it; O stays far inside fp32 range), so a key tens of exp2
// units above the reference costs nothing extra, and O / l is exact
// whatever reference was used.
//
// LDS rows are padded by 16 bytes instead of XOR-swizzled: gfx950 serves a
// 16-byte-per-lane read 16 lanes at a time over a 256-byte bank window, and a
// row stride of 17 (K) or 9 (V^T) 16-byte slots puts the 16 rows read together
// in 16 distinct slots, while every fragment sits at a constant offset from
// one per-lane base address.
constexpr float kGuardP = 18446744073709551616.0f;   // 2^64: largest accepted sum of a lane's 32 weights of a tile
constexpr int KROW = DH + 8;     // K tile row: 128 dh + 8 pad elements (272 B)
constexpr int VROW = KT + 8;     // V^T tile row: 64 keys + 8 pad elements (144 B)

__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(const uint16_t* __restrict__ q,
                                                           const int32_t* __restrict__ idx,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, int kq,
                                                           int n, int Hq, int Hkv, float sl2,
                                                           uint16_t* __restrict__ o) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[3][KT * KROW];   // K_t stays for its whole step t
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
  // The block's key range comes from the smallest and largest row among its
  // 64 queries (idx need not be sorted): each lane reads two of them and the
  // wave reduces.  Rows past kq repeat the last query's row.
  int kmin, kmax;
  {
    const int ra = idx[min(q0 + l32, kq - 1)], rb = idx[min(q0 + 32 + l32, kq - 1)];
    kmin = min(ra, rb);
    kmax = max(ra, rb);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      kmin = min(kmin, __shfl_xor(kmin, o));
      kmax = max(kmax, __shfl_xor(kmax, o));
    }
  }
  const int ntiles = kmax / KT + 1;
  const int nfull = (kmin + 1) / KT;                // tiles entirely below every query of the block

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
  // two register sets: a step stores the tiles loaded one step earlier and
  // loads the next ones, so every load has two steps to land
  u32x4 kra[2], vra[2], krb[2], vrb[2];
  auto load_k = [&](u32x4 (&kr)[2], int j0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = min(j0 + (tid >> 4) + 32 * i, n - 1);
      kr[i] = ld16(kbase + j * row_stride);
    }
  };
  auto load_v = [&](u32x4 (&vr)[2], int j0) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = min(j0 + 2 * kp + e, n - 1);
      vr[e] = ld16(vbase + j * row_stride);
    }
  };
  auto store_k = [&](const u32x4 (&kr)[2], int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) st16(Ks[buf] + ((tid >> 4) + 32 * i) * KROW + (tid & 15) * 8, kr[i]);
  };
  auto store_v = [&](const u32x4 (&vr)[2], int buf) {
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
  // mask tile t's keys beyond each query; key of reg r = t*64 + kt*32 +
  // (r>>3)*16 + half*8 + (r&7)
  auto mask = [&](int t, f32x16 (&sd)[2]) {
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
  };
  // P_t = exp2(logit * scale * log2e - m_ref) as bf16 MFMA operands; returns
  // this half-wave's sum of the tile's weights (not yet added to l)
  auto softmax = [&](f32x16 (&sc)[2], bf16x8 (&pc)[4]) {
    float a[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kt][sub * 8 + e], sl2, -m_ref));
          const int i = kt * 16 + sub * 8 + e;
          a[i & 3] = i < 4 ? pv[e] : a[i & 3] + pv[e];
        }
        pc[kt * 2 + sub] = __builtin_convertvector(pv, bf16x8);
      }
    return (a[0] + a[1]) + (a[2] + a[3]);
  };
  // Accept tile t's weights, or, when some lane's sum left [0, 2^64] (a
  // logit 64 units above the reference, or a NaN), move the
  // reference to the exact running max (shared by the two half-waves of a
  // query), rescale O and l, and form the tile's P again.  O already holds
  // P_{t-1} V_{t-1} at the old reference, so nothing else is pending.
  // The logits of tile t are formed again from K_t, still in Ks[t % 3]
  // during step t, so they need not stay in registers past the softmax.
  auto settle = [&](int t, bf16x8 (&pc)[4], float ts) {
    if (__builtin_expect(__any(!(ts <= kGuardP)), 0)) {
      f32x16 sc[2];
      logits(t % 3, sc);
      mask(t, sc);
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sc[kt][r]);
      mx *= sl2;
      const float m_new = fmaxf(m_ref, fmaxf(mx, __shfl_xor(mx, 32)));
      const float alpha = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
      m_ref = m_new;
      ts = softmax(sc, pc);
    }
    l_part += ts;
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
  // trails K by two tiles: step t stores K_{t+2} (into K buffer (t+2) % 3)
  // and V_t (into V buffer t & 1) from the registers kc / vc loaded during
  // step t-1, and loads V_{t+1} and K_{t+3} into kn / vn; V_t is read at step
  // t+1.
  auto step = [&](auto with_pv, int t, f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pp)[4],
                  bf16x8 (&pc)[4], u32x4 (&kc)[2], u32x4 (&vc)[2], u32x4 (&kn)[2], u32x4 (&vn)[2]) {
    constexpr bool kPV = decltype(with_pv)::value;
    // K/V staging is unconditional (rows clamp to n-1; past the last tile the
    // K store lands in buffer (t+2) % 3, whose tile was read in step t-2), so
    // no branch splits the MFMA / VALU block
    load_k(kn, (t + 3) * KT);
    load_v(vn, (t + 1) * KT);
    logits((t + 1) % 3, sn);             // stale data past the last tile; unused
    if constexpr (kPV) pv_mma((t - 1) & 1, pp);
    float ts = softmax(sc, pc);
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
    asm volatile("" : "+v"(pc[0]), "+v"(pc[1]), "+v"(pc[2]), "+v"(pc[3]), "+v"(ts));
    settle(t, pc, ts);
    store_k(kc, (t + 2) % 3);
    store_v(vc, t & 1);
    if (t + 1 < ntiles) mask(t + 1, sn);
    __syncthreads();
  };

  // prologue: K_0, K_1 staged; K_2 and V_0 in registers (set a) for step 0
  // to store; logits of tile 0
  load_k(kra, 0);
  store_k(kra, 0);
  if (ntiles > 1) {
    load_k(kra, KT);
    store_k(kra, 1);
  }
  load_k(kra, 2 * KT);
  load_v(vra, 0);
  __syncthreads();                        // K_0, K_1 in LDS
  f32x16 sa[2], sb[2];
  bf16x8 pa[4], pb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    pa[c] = bf16x8{};
    pb[c] = bf16x8{};
  }
  logits(0, sa);
  mask(0, sa);
  // tile 0's reference: its exact max (key 0 is visible to every query), so
  // the first tile is not formed twice
  {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sa[kt][r]);
    m_ref = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
  }
  step(std::false_type{}, 0, sa, sb, pb, pa, kra, vra, krb, vrb);
  int t = 1;
  for (; t + 1 < ntiles; t += 2) {
    step(std::true_type{}, t, sb, sa, pa, pb, krb, vrb, kra, vra);
    step(std::true_type{}, t + 1, sa, sb, pb, pa, kra, vra, krb, vrb);
  }
  if (t < ntiles) step(std::true_type{}, t, sb, sa, pa, pb, krb, vrb, kra, vra);
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
// Two passes over the keys, both on v_mfma_f32_32x32x16_bf16 with 64-key K
// tiles in LDS shared by the waves of a workgroup.  A workgroup is (key
// chunk, group of 4 query heads that share one KV head); each of its waves
// holds the queries of 32*PT probes of one head in registers, and
// P / (32*PT) waves per head cover all P probes (8 waves at P = 128, so no
// wave holds more than 64 probes' queries).
//
// K tiles stream straight from global memory into a ring of NS LDS stages
// (global_load_lds, the swizzle applied on the global side), NS-1 tiles
// ahead of the one being scored: one tile in flight per workgroup left the
// passes waiting on load latency.
//
// Pass 1 (stats): per (chunk, head, probe) a reference and the sum of
// exp2(scale*log2e * logit - reference), logits as S^T = K Q^T so a lane owns
// a probe.  The reference is set from the exact max only when a 16-logit
// chain's sum of weights leaves [0, 2^64], so a logit costs one fma, one exp
// and one add, with no max.
// Combine: per (head, probe) the chunk partials merge into
// M = max + log2(sum).
// Pass 2 (column sums): logits as S = Q K^T so a lane owns a key, and each
// logit adds exp2(scale*log2e * logit - M) = its softmax weight to its key's
// sum: one fma, one exp and one add per logit.  The head quad's sums are
// added in a fixed order in LDS; a last launch adds the head quads in a
// fixed order.  Causal masking is applied only to the tiles that reach past
// the first probe row (the last one or two tiles of the sequence).  No float
// atomics: the result does not depend on scheduling.
//
// A key chunk is a multiple of the 64-key tile of at least 128 keys: the
// shortest whose grid of chunks x head quads fits one round of resident
// workgroups.  A partly filled second round costs a whole chunk's time, while
// every workgroup also loads its probes' queries, so chunks stay as long as
// that round allows; past max_chunk keys the grid runs in several rounds.
constexpr int MIN_CHUNK = 128;
constexpr float kProbeGuard = 18446744073709551616.0f;   // 2^64: largest accepted sum of 16 weights
constexpr int NS = 4;                // K tile stages in LDS

// Longest key chunk of pass 2 (its column sums sit in LDS): 32 KiB of sums
// beside the 64 KiB K ring at one workgroup per CU, 8 KiB at two.
constexpr int max_chunk(int occ) { return occ == 1 ? 8192 : 2048; }

// Keys per chunk: the shortest multiple of 64 whose grid fits one round of
// resident workgroups, so each workgroup loads its probe queries and fills its
// K ring once per CU (4096-key chunks at 131072 keys and 128 probes: 333 us
// per call against 373 us with 1024-key chunks in four rounds).
int probe_chunk(int n, int Hq, int occ) {
  const long slots = 256L * occ;                                   // resident workgroups
  const long need = ((long)n * (Hq / 4) + slots - 1) / slots;      // keys per chunk for one round
  const long c = ((need + KT - 1) / KT) * KT;
  return c < MIN_CHUNK ? MIN_CHUNK : (int)(c > max_chunk(occ) ? max_chunk(occ) : c);
}

// Issue the global -> LDS copy of the K tile [64 keys][128] of KV head g at
// key j0 into `stage`, NT threads.  Instruction i of wave w fills the 1 KiB
// block of keys 4*blk .. 4*blk+3 (blk = w*PER + i): lane L writes physical
// chunk L%16 of key 4*blk + L/16, so it fetches logical chunk
// (L%16) ^ (key & 15) -- the kswz swizzle, applied on the global side.  Keys
// >= n clamp to n-1 (always masked).
template <int NT>
__device__ __forceinline__ void issue_k_tile(uint16_t* stage, const uint16_t* k, int j0, int n, int Hkv, int g,
                                             int tid) {
  constexpr int PER = 16 / (NT / 64);   // 1 KiB blocks per wave
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int blk = wave * PER + i;
    const int key = blk * 4 + (lane >> 4);
    const int lch = (lane & 15) ^ (key & 15);
    int j = j0 + key;
    j = j < n ? j : n - 1;
    const uint16_t* src = k + (long)j * Hkv * DH + g * DH + lch * 8;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(stage + blk * 512), 16, 0, 0);
  }
}

// Workgroup barrier once at most `tiles` K-tile copies of this thread are
// still in flight: s_waitcnt on vmcnt (the copies are counted in issue
// order) and on lgkmcnt (this wave's LDS stores), then s_barrier.  A plain
// __syncthreads would also wait for every copy still in flight.
template <int NT>
__device__ __forceinline__ void barrier_k_tiles(int tiles) {
  constexpr int PER = 16 / (NT / 64);
  static_assert(PER * (NS - 2) < 16, "vmcnt field");
  if (tiles >= 2) __builtin_amdgcn_s_waitcnt(0x0070 | (2 * PER));
  else if (tiles == 1) __builtin_amdgcn_s_waitcnt(0x0070 | PER);
  else __builtin_amdgcn_s_waitcnt(0x0070);
  __builtin_amdgcn_s_barrier();
}

template <int PT>
__device__ __forceinline__ void load_probe_q(bf16x8 (&qf)[PT][8], const uint16_t* q, int pbase, int Hq, int h,
                                             int l32, int half) {
#pragma unroll
  for (int c = 0; c < PT; ++c)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[c][kk] = *reinterpret_cast<const bf16x8*>(q + ((long)(pbase + c * 32 + l32) * Hq + h) * DH + kk * 16 +
                                                   half * 8);
}

// each wave: 32*PT probes of one head; PW waves per head; P = 32*PT*PW; OCC workgroups per CU
template <int PT, int PW, int OCC>
__global__ __launch_bounds__(256 * PW, OCC) void probe_stats_kernel(const uint16_t* __restrict__ q,
                                                                       const uint16_t* __restrict__ k, int n,
                                                                       int chunk_keys, int Hq, int Hkv, float sl2,
                                                                       float* __restrict__ part_lse, int nchunks) {
  constexpr int P = 32 * PT * PW, NT = 256 * PW;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NS][KT * DH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int h = blockIdx.y * 4 + (wave & 3);
  const int pbase = (wave >> 2) * 32 * PT;            // this wave's first probe
  const int g = (blockIdx.y * 4) / (Hq / Hkv);
  const int chunk = blockIdx.x;
  const int c0 = chunk * chunk_keys;
  const int nt = min(chunk_keys / KT, (n - c0 + KT - 1) / KT);   // key tiles of this chunk
  const int first_probe_row = n - P;

  bf16x8 qf[PT][8];
  load_probe_q<PT>(qf, q, pbase, Hq, h, l32, half);
  // no wait here: the queries are older than every K copy, so the first
  // ring barrier's in-order count also covers them
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nt) issue_k_tile<NT>(Ks[s], k, c0 + s * KT, n, Hkv, g, tid);
  float m[PT], l[PT];
#pragma unroll
  for (int c = 0; c < PT; ++c) { m[c] = -INFINITY; l[c] = 0.f; }

  // one tile's logits added to each probe's running sum against the lane's
  // reference m[c] (exp2 units), 32 keys at a time (the K fragments of those
  // keys are shared by the PT probe tiles).  There is no per-logit max: the
  // sum of a chain's 16 weights is tested instead, and a wave in which some
  // lane's sum leaves [0, 2^64] (no reference yet, a logit 64 units above
  // the reference, or a NaN) redoes that chain against the exact running max,
  // which becomes the reference.  A sum below 2^64 keeps l far from overflow,
  // and any reference gives the same M = ref + log2(l) up to rounding.
  // MASK: the tile reaches past the first probe row (causal mask per key).
  auto tile = [&](auto mask, const uint16_t* kt_s, int j0) {
    constexpr bool MASK = decltype(mask)::value;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bf16x8 kf[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8*>(kt_s + kswz(kt * 32 + perm32(l32), kk * 2 + half));
#pragma unroll
      for (int c = 0; c < PT; ++c) {
        f32x16 s;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) s = mfma32x32x16(kf[kk], qf[c][kk], kk == 0 ? f32x16{} : s);
        if constexpr (MASK) {
          // reg r holds key j0 + kt*32 + (r>>3)*16 + half*8 + (r&7)
          const int prow = first_probe_row + pbase + c * 32 + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (j0 + kt * 32 + (r >> 3) * 16 + half * 8 + (r & 7) > prow) s[r] = -INFINITY;
        }
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        const float nm = -m[c];
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          a0 += __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, nm));
          a1 += __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], sl2, nm));
          a2 += __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 2], sl2, nm));
          a3 += __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 3], sl2, nm));
        }
        const float ts = (a0 + a1) + (a2 + a3);
        if (__builtin_expect(__any(!(ts <= kProbeGuard)), 0)) {
          float mx = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[r]);
          const float mref = __builtin_fmaxf(m[c], mx * sl2);
          const float alpha = mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[c] - mref);
          const float mz = mref == -INFINITY ? 0.f : mref;   // a lane with no visible key yet adds zeros
          float b0 = 0.f, b1 = 0.f;
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            b0 += __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -mz));
            b1 += __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], sl2, -mz));
          }
          l[c] = l[c] * alpha + (b0 + b1);
          m[c] = mref;
        } else {
          l[c] += ts;
        }
      }
    }
  };

  // Tiles entirely below the first probe row (all but the sequence's last one
  // or two) run software-pipelined across the ring barriers: the weights of
  // each 16-logit chain are formed while the matrix core computes the next
  // chain, and a tile's last chain is finished under the next tile's first.
  auto chain = [&](const bf16x8 (&kf)[8], int c) {
    f32x16 s;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = mfma32x32x16(kf[kk], qf[c][kk], kk == 0 ? f32x16{} : s);
    return s;
  };
  auto wsum = [&](const f32x16& s, int c) {
    const float nm = -m[c];
    float a[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, nm));
      a[r & 3] = r < 4 ? w : a[r & 3] + w;
    }
    return (a[0] + a[1]) + (a[2] + a[3]);
  };
  // accept a chain's sum, or redo the chain against the exact running max
  auto settle = [&](const f32x16& s, int c, float ts) {
    if (__builtin_expect(__any(!(ts <= kProbeGuard)), 0)) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[r]);
      const float mref = __builtin_fmaxf(m[c], mx * sl2);
      const float alpha = mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[c] - mref);
      const float mz = mref == -INFINITY ? 0.f : mref;
      float b0 = 0.f, b1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        b0 += __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -mz));
        b1 += __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], sl2, -mz));
      }
      l[c] = l[c] * alpha + (b0 + b1);
      m[c] = mref;
    } else {
      l[c] += ts;
    }
  };
  // one MFMA, then six VALU instructions, eight times: a chain's MFMAs
  // interleaved with the previous chain's weights
  auto interleave = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
    }
  };
  // chains of a tile in the order i = kt*PT + c; sp carries the last one
  auto tile_pipe = [&](auto first, const uint16_t* kt_s, f32x16& sp) {
    constexpr bool FIRST = decltype(first)::value;
    bf16x8 kf[2][8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        kf[kt][kk] = *reinterpret_cast<const bf16x8*>(kt_s + kswz(kt * 32 + perm32(l32), kk * 2 + half));
    f32x16 sc[2 * PT];
#pragma unroll
    for (int i = 0; i < 2 * PT; ++i) {
      sc[i] = chain(kf[i / PT], i % PT);
      if (i == 0) {
        if constexpr (!FIRST) {
          const float ts = wsum(sp, PT - 1);
          interleave();
          settle(sp, PT - 1, ts);
        }
      } else {
        const float ts = wsum(sc[i - 1], (i - 1) % PT);
        interleave();
        settle(sc[i - 1], (i - 1) % PT, ts);
      }
    }
    sp = sc[2 * PT - 1];
  };

  int nt_fast = first_probe_row + 1 - c0;            // keys of the chunk at or below the first probe row
  nt_fast = nt_fast <= 0 ? 0 : min(nt, nt_fast / KT);
  f32x16 sp;
  for (int t = 0; t < nt; ++t) {
    const int j0 = c0 + t * KT;
    // every thread's copies of tile t have landed; stage (t-1) % NS is free
    barrier_k_tiles<NT>(min(NS - 2, nt - 1 - t));
    if (t + NS - 1 < nt) issue_k_tile<NT>(Ks[(t + NS - 1) % NS], k, j0 + (NS - 1) * KT, n, Hkv, g, tid);
    if (t < nt_fast) {
      if (t == 0) tile_pipe(std::true_type{}, Ks[t % NS], sp);
      else tile_pipe(std::false_type{}, Ks[t % NS], sp);
    } else {
      if (t == nt_fast && t > 0) settle(sp, PT - 1, wsum(sp, PT - 1));
      tile(std::true_type{}, Ks[t % NS], j0);        // reaches past the first probe row
    }
  }
  if (nt_fast == nt && nt > 0) settle(sp, PT - 1, wsum(sp, PT - 1));
  // merge the two half-waves (they hold different keys of the same probes)
  // and store the chunk's log-sum-exp ref + log2(sum) (exp2 units; -inf when
  // no key of the chunk is visible to the probe), the chunks of one (head,
  // probe) row side by side
#pragma unroll
  for (int c = 0; c < PT; ++c) {
    const float m2 = __shfl_xor(m[c], 32), l2 = __shfl_xor(l[c], 32);
    const float mt = fmaxf(m[c], m2);
    float lse = -INFINITY;
    if (mt != -INFINITY) lse = mt + log2f(l[c] * exp2f(m[c] - mt) + l2 * exp2f(m2 - mt));
    if (half == 0) part_lse[((long)h * P + pbase + c * 32 + l32) * nchunks + chunk] = lse;
  }
}

// Combine the chunks' log-sum-exps -> per (head, probe) M = log2 of the sum
// over chunks of 2^lse (exp2 units), taken against the largest.  One wave per
// (head, probe), whose chunks lie side by side; lanes stride over chunks,
// fixed-order wave tree.
__global__ __launch_bounds__(256) void probe_combine_kernel(const float* __restrict__ part_lse, int nchunks,
                                                            int HP, float* __restrict__ fin_M) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= HP) return;
  const float* row = part_lse + (long)i * nchunks;
  float mt = -INFINITY;
  for (int c = lane; c < nchunks; c += 64) mt = fmaxf(mt, row[c]);
  mt = wave_max(mt);
  float lt = 0.f;
  for (int c = lane; c < nchunks; c += 64) {
    const float v = row[c];
    if (v != -INFINITY) lt += exp2f(v - mt);
  }
  lt = wave_sum(lt);
  if (lane == 0) fin_M[i] = mt + log2f(lt);
}

// Pass 2: column sums of the normalised probe softmax for one key chunk and
// one head quad; logits formed as S = Q K^T so a lane owns one key, and each
// lane keeps -M of its 16*PT probe rows in registers.  Per tile, each wave
// adds its two half-waves and leaves its 64 key sums in LDS; after the next
// tile's ring barrier one wave adds the waves' sums in a fixed order into the
// chunk's column sums, also in LDS, which are written out once at the end.
template <int PT, int PW, int OCC>
__global__ __launch_bounds__(256 * PW, OCC) void probe_colsum_kernel(const uint16_t* __restrict__ q,
                                                                        const uint16_t* __restrict__ k, int n,
                                                                        int chunk_keys, int Hq, int Hkv, float sl2,
                                                                        const float* __restrict__ fin_M,
                                                                        float* __restrict__ quad_sum) {
  constexpr int P = 32 * PT * PW, NT = 256 * PW, NW = 4 * PW;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NS][KT * DH];
  __shared__ __attribute__((aligned(16))) float red[2][KT][NW];     // [key][wave]
  __shared__ __attribute__((aligned(16))) float csum[max_chunk(OCC)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int h = blockIdx.y * 4 + (wave & 3);
  const int pbase = (wave >> 2) * 32 * PT;
  const int g = (blockIdx.y * 4) / (Hq / Hkv);
  const int chunk = blockIdx.x;
  const int c0 = chunk * chunk_keys;
  const int nt = min(chunk_keys / KT, (n - c0 + KT - 1) / KT);
  const int first_probe_row = n - P;

  // -M of this lane's rows: reg r of probe tile c is probe pbase + c*32 + (r>>2)*8 + half*4 + (r&3)
  float nM[PT][16];
#pragma unroll
  for (int c = 0; c < PT; ++c)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const f32x4 mm = *reinterpret_cast<const f32x4*>(fin_M + (long)h * P + pbase + c * 32 + qd * 8 + half * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) nM[c][qd * 4 + e] = -mm[e];
    }
  bf16x8 qf[PT][8];
  load_probe_q<PT>(qf, q, pbase, Hq, h, l32, half);
  // no wait here: the queries and M are older than every K copy, so the
  // first ring barrier's in-order count also covers them
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nt) issue_k_tile<NT>(Ks[s], k, c0 + s * KT, n, Hkv, g, tid);

  // one tile's softmax weights summed per key (lane = key); MASK: the tile
  // reaches past the first probe row
  auto tile = [&](auto mask, const uint16_t* kt_s, int j0, float (&cs)[2]) {
    constexpr bool MASK = decltype(mask)::value;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = j0 + kt * 32 + perm32(l32);          // this lane's key column
      bf16x8 kf[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8*>(kt_s + kswz(kt * 32 + perm32(l32), kk * 2 + half));
      float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < PT; ++c) {
        f32x16 s;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) s = mfma32x32x16(qf[c][kk], kf[kk], kk == 0 ? f32x16{} : s);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float w = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, nM[c][r]));
          if constexpr (MASK) {
            const int row = pbase + c * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            w = key > first_probe_row + row ? 0.f : w;
          }
          a[r & 3] += w;
        }
      }
      cs[kt] = (a[0] + a[1]) + (a[2] + a[3]);
    }
  };
  // the waves' sums of tile u, added in wave order, into the chunk's sums
  auto reduce = [&](int u) {
    if (tid < KT) {
      const float* rr = red[u & 1][tid];
      float tot = rr[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) tot += rr[w];
      csum[u * KT + tid] = tot;
    }
  };
  // this wave's sums of tile u (both half-waves added) into red[u & 1]
  auto put = [&](int u, float cs0, float cs1) {
    cs0 += __shfl_xor(cs0, 32);
    cs1 += __shfl_xor(cs1, 32);
    if (half == 0) {
      red[u & 1][perm32(l32)][wave] = cs0;
      red[u & 1][32 + perm32(l32)][wave] = cs1;
    }
  };
  auto raw_barrier = []() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0): LDS traffic done (vmcnt untouched)
    __builtin_amdgcn_s_barrier();
  };

  // Tiles entirely below the first probe row run software-pipelined across
  // the ring barriers, as in the stats pass: a chain's weights are formed
  // while the matrix core computes the next chain.  A tile's last chain is
  // finished under the next tile's first, so its sums reach red one tile
  // later and are reduced two tiles later.
  auto chain = [&](const bf16x8 (&kf)[8], int c) {
    f32x16 s;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) s = mfma32x32x16(qf[c][kk], kf[kk], kk == 0 ? f32x16{} : s);
    return s;
  };
  auto wadd = [&](const f32x16& s, int c, float (&a)[4], bool init) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, nM[c][r]));
      a[r & 3] = (init && r < 4) ? w : a[r & 3] + w;
    }
  };
  auto interleave = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
    }
  };
  // sl: last chain of the previous tile; a1p: that tile's kt = 1 partial
  // sums (its chains before the last); cs0p: its finished kt = 0 sum
  auto tile_pipe = [&](auto first, int t, const uint16_t* kt_s, f32x16& sl, float (&a1p)[4], float& cs0p) {
    constexpr bool FIRST = decltype(first)::value;
    // the kt = 1 fragments are read after the first chain is issued (fewer live registers)
    bf16x8 kf[2][8];
    auto frags = [&](int kt) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        kf[kt][kk] = *reinterpret_cast<const bf16x8*>(kt_s + kswz(kt * 32 + perm32(l32), kk * 2 + half));
    };
    frags(0);
    float a0[4], a1[4];
    f32x16 sc[2 * PT];
#pragma unroll
    for (int i = 0; i < 2 * PT; ++i) {
      sc[i] = chain(kf[i / PT], i % PT);
      if (i == 0) frags(1);
      if (i == 0) {
        if constexpr (!FIRST) {
          wadd(sl, PT - 1, a1p, PT == 1);
          interleave();
          put(t - 1, cs0p, (a1p[0] + a1p[1]) + (a1p[2] + a1p[3]));
        }
      } else {
        const int j = i - 1;                       // chain j = kt*PT + c
        if (j / PT == 0) wadd(sc[j], j % PT, a0, j % PT == 0);
        else wadd(sc[j], j % PT, a1, j % PT == 0);
        interleave();
      }
    }
    cs0p = (a0[0] + a0[1]) + (a0[2] + a0[3]);
    if constexpr (PT > 1) {                        // with one probe tile, the next wadd starts a1p
#pragma unroll
      for (int e = 0; e < 4; ++e) a1p[e] = a1[e];
    }
    sl = sc[2 * PT - 1];
  };

  int nt_fast = first_probe_row + 1 - c0;
  nt_fast = nt_fast <= 0 ? 0 : min(nt, nt_fast / KT);
  if (nt_fast > 0) {
    f32x16 sl;
    float a1p[4] = {0.f, 0.f, 0.f, 0.f}, cs0p = 0.f;
    for (int t = 0; t < nt_fast; ++t) {
      // tile t in LDS; stage (t-1) % NS free; every wave's sums of tile t-2 in red[t & 1]
      barrier_k_tiles<NT>(min(NS - 2, nt - 1 - t));
      if (t >= 2) reduce(t - 2);
      if (t + NS - 1 < nt) issue_k_tile<NT>(Ks[(t + NS - 1) % NS], k, c0 + (t + NS - 1) * KT, n, Hkv, g, tid);
      if (t == 0) tile_pipe(std::true_type{}, t, Ks[t % NS], sl, a1p, cs0p);
      else tile_pipe(std::false_type{}, t, Ks[t % NS], sl, a1p, cs0p);
    }
    wadd(sl, PT - 1, a1p, PT == 1);
    put(nt_fast - 1, cs0p, (a1p[0] + a1p[1]) + (a1p[2] + a1p[3]));
    raw_barrier();
    if (nt_fast >= 2) reduce(nt_fast - 2);
    reduce(nt_fast - 1);
    raw_barrier();
  }
  // tiles that reach past the first probe row: no pipelining, sums reduced one tile later
  for (int t = nt_fast; t < nt; ++t) {
    const int j0 = c0 + t * KT;
    barrier_k_tiles<NT>(min(NS - 2, nt - 1 - t));
    if (t > nt_fast) reduce(t - 1);
    if (t + NS - 1 < nt) issue_k_tile<NT>(Ks[(t + NS - 1) % NS], k, j0 + (NS - 1) * KT, n, Hkv, g, tid);
    float cs[2];
    tile(std::true_type{}, Ks[t % NS], j0, cs);
    put(t, cs[0], cs[1]);
  }
  if (nt_fast < nt) {
    raw_barrier();
    reduce(nt - 1);
  }
  __syncthreads();
  const int nk = min(nt * KT, n - c0);
  for (int i = tid; i < nk; i += NT) quad_sum[(long)blockIdx.y * n + c0 + i] = csum[i];
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
  // part_lse [HP][nchunks]; fin_M [HP] (2*HP reserved); quad_sum [Hq/4 * n]
  size_t b = HP * nchunks * 4 + 2 * HP * 4 + (size_t)((Hq + 3) / 4) * n * 4;
  return (b + 255) & ~(size_t)255;
}

// The two passes and the chunk combine for P = 32*PT*PW probes.
template <int PT, int PW, int OCC>
void probe_passes(const uint16_t* q, const uint16_t* k, int n, int Hq, int Hkv, float sl2, void* ws,
                  float* scores, hipStream_t s) {
  constexpr int P = 32 * PT * PW;
  const int ck = probe_chunk(n, Hq, OCC);
  const int nchunks = (n + ck - 1) / ck;
  const long HP = (long)Hq * P;
  float* part_lse = reinterpret_cast<float*>(ws);
  float* fin_M = part_lse + HP * nchunks;
  float* quad = fin_M + 2 * HP;
  const dim3 grid(nchunks, Hq / 4);
  hipLaunchKernelGGL((probe_stats_kernel<PT, PW, OCC>), grid, dim3(256 * PW), 0, s, q, k, n, ck, Hq, Hkv, sl2,
                     part_lse, nchunks);
  hipLaunchKernelGGL(probe_combine_kernel, dim3((HP + 3) / 4), dim3(256), 0, s, part_lse, nchunks, (int)HP, fin_M);
  hipLaunchKernelGGL((probe_colsum_kernel<PT, PW, OCC>), grid, dim3(256 * PW), 0, s, q, k, n, ck, Hq, Hkv, sl2,
                     fin_M, quad);
  hipLaunchKernelGGL(quad_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, quad, Hq / 4, n, scores);
}

hipError_t launch_probe_bf16(const uint16_t* q, const uint16_t* k, int n, int P, int Hq, int Hkv,
                             float scale, float* scores, void* ws, hipStream_t s) {
  const float sl2 = scale * kLog2e;
  // Two waves per SIMD, 64 probes per wave: at 64 probes two 4-wave
  // workgroups per CU (one wave per head), at 128 one 8-wave workgroup (two
  // waves per head).  One 128-probe wave per SIMD and four 32-probe waves
  // per SIMD both measured slower.
  switch (P) {
    case 32: probe_passes<1, 1, 2>(q, k, n, Hq, Hkv, sl2, ws, scores, s); break;
    case 64: probe_passes<2, 1, 2>(q, k, n, Hq, Hkv, sl2, ws, scores, s); break;
    case 128: probe_passes<2, 2, 1>(q, k, n, Hq, Hkv, sl2, ws, scores, s); break;
    default: return hipErrorInvalidValue;
  }
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
