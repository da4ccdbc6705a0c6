// Top-k token selection with forced probe rows, gfx950.
//
// Scores (or the MaxNorm-Add or Multiply fusion of two scores) are mapped to unsigned
// keys whose integer order is the float order (NaN lowest, -0 == +0).  An
// MSB-first radix select over the non-forced rows finds the threshold key T
// of the (k - n_forced)-th largest and how many rows equal to T to take; a
// ballot compaction in index order then writes exactly k ascending indices:
// forced rows, rows above T, and the lowest-index rows equal to T.
//
// Up to 32K scores one 1024-thread workgroup does the whole selection with
// the keys in registers (the call is bound by latency, not bandwidth; above
// 32K the selection spreads over many workgroups, see mtopk_* below).  Wave
// w owns the contiguous rows [w*C, (w+1)*C) and its lanes walk them 64 at a
// time, so every load is one coalesced 256-byte access.  The radix passes
// skip the leading key bits that all free rows share (found by an OR/AND
// reduction).  The first digit is 11 bits wide and is counted in one shared
// 2048-bin histogram.  When the bin holding the threshold has at most CAP keys
// (the usual case), those keys are copied to LDS and a single wave finishes
// the remaining digits over them, with no workgroup barrier per digit; a
// larger bin (many equal scores) continues with 8-bit workgroup passes.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace spts {
namespace {

constexpr int TPB = 1024;
constexpr int NW = TPB / 64;
constexpr int B1 = 11;                 // width of the first digit
constexpr int NB1 = 1 << B1;           // its histogram bins
constexpr int CAP = 8192;              // keys a single wave finishes from LDS

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;                 // NaN ranks below everything
  if (f == 0.0f) f = 0.0f;               // -0 -> +0
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// MaxNorm-Add in fp32 with a fixed operation order (no contraction); Multiply
// is one fp32 product.
__device__ __forceinline__ float fuse(float a, float b, float ma, float mb, float wa, float wb) {
  const float ta = ma > 0.f ? __fmul_rn(wa, __fdiv_rn(a, ma)) : 0.f;
  const float tb = mb > 0.f ? __fmul_rn(wb, __fdiv_rn(b, mb)) : 0.f;
  return __fadd_rn(ta, tb);
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Wave-wide inclusive scans on DPP (no LDS round trip): Hillis-Steele within
// each 16-lane row (row_shr 1, 2, 4, 8), then row_bcast:15 carries row 0's and
// row 2's totals into rows 1 and 3, and row_bcast:31 carries rows 0-1 into
// rows 2-3.  A lane whose source is outside its row, or whose row is masked
// off, receives the operation's identity.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v, uint32_t id, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xa, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xc, 0xf, false));
  return v;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  return (int)wave_scan_dpp((uint32_t)v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ int wave_sum_int(int v) { return __builtin_amdgcn_readlane(wave_incl_scan(v), 63); }

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_dpp(v, 0u, [](uint32_t a, uint32_t b) { return a | b; }), 63);
}

__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane(
      (int)wave_scan_dpp(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a & b; }), 63);
}

__device__ __forceinline__ float wave_fmax(float v) {
  const uint32_t r = wave_scan_dpp(__float_as_uint(v), __float_as_uint(-INFINITY), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  });
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
}

// maxima of a and b over the workgroup (fmaxf: NaN is ignored), one barrier pair
__device__ void block_max2(float a, float b, float* sh, float& ma, float& mb) {
  a = wave_fmax(a);
  b = wave_fmax(b);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { sh[w] = a; sh[NW + w] = b; }
  __syncthreads();
  ma = -INFINITY;
  mb = -INFINITY;
  for (int i = 0; i < NW; ++i) { ma = fmaxf(ma, sh[i]); mb = fmaxf(mb, sh[NW + i]); }
  __syncthreads();
}

// Suffix search over NB bins held NB/64 per lane, highest digit first (lane t
// holds bins NB-1-t*(NB/64) downwards): the digit d holding the rem-th
// largest key, how many keys lie above that digit's bin and the bin's count.
// Called by one whole wave; the result is valid in every lane.
template <int NB>
__device__ __forceinline__ void wave_find_digit(const int* h, int rem, int lane, int& d, int& above, int& cnt) {
  constexpr int PER = NB / 64;
  const int top = NB - 1 - lane * PER;
  int part = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) part += h[top - q];
  const int incl = wave_incl_scan(part);
  const int excl = incl - part;
  const bool mine = excl < rem && rem <= incl;
  int dd = 0, ab = 0, cc = 0;
  if (mine) {
    ab = excl;
    for (int q = 0; q < PER; ++q) {
      const int c = h[top - q];
      if (ab + c >= rem) { dd = top - q; cc = c; break; }
      ab += c;
    }
  }
  const int src = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)__ballot(mine)) - 1);
  d = __builtin_amdgcn_readlane(dd, src);
  above = __builtin_amdgcn_readlane(ab, src);
  cnt = __builtin_amdgcn_readlane(cc, src);
}

// Each lane keeps the keys of its IPT rows in registers across all passes
// (n <= 1024 * IPT); larger selections run on many workgroups (mtopk_* below).
template <int IPT>
__global__ __launch_bounds__(TPB) void topk_kernel(const float* __restrict__ s_a,
                                                   const float* __restrict__ s_b, float wa, float wb,
                                                   int mult, int n, int k, int nf, int32_t* __restrict__ idx,
                                                   float* __restrict__ fused_out, long s_stride,
                                                   long idx_stride) {
  static_assert(IPT > 0, "keys per lane");
  // Every per-key update below is unconditional: a row that does not count
  // goes to a dummy slot of its own lane (index + lane past the end), so the
  // loops carry no branches and the dummies never collide.
  __shared__ int hist1[NB1 + 64];        // first digit
  __shared__ uint32_t pool[CAP + 64];    // candidate keys, or the per-wave histograms of the fallback passes
  __shared__ int h8[256 + 64];           // the finishing wave's histogram
  __shared__ int tot_hist[256];
  __shared__ float red[2 * NW];
  __shared__ uint32_t bits_sh[2][NW];
  __shared__ int cnt_sh[2][NW];
  __shared__ int sel[3];
  __shared__ int ccount;
  int (*hist)[320] = reinterpret_cast<int (*)[320]>(pool);   // [NW][256 + 64] fallback, one per wave
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  s_a += (long)blockIdx.x * s_stride;    // batched rows (a single call: one workgroup, offsets 0)
  idx += (long)blockIdx.x * idx_stride;

  if (k >= n) {
    for (int i = tid; i < n; i += TPB) idx[i] = i;
    if (!(fused_out && s_b)) return;
  }

  float ma = 0.f, mb = 0.f;                   // MaxNorm-Add maxima, from the loaded rows below
  constexpr int UNROLL_J = IPT;
  const int nfree = n - nf;
  constexpr int J = IPT;                      // rows per lane
  const int base = w * J * 64 + lane;                  // row of (w, j, lane) = base + 64 j
  // a lane's rows base + 64 j are valid (< n) for j < jv and free (< nfree)
  // for j < jf; loops test j against these instead of keeping a mask per row
  int jv = n > base ? (n - base + 63) / 64 : 0;
  int jf = nfree > base ? (nfree - base + 63) / 64 : 0;
  // an empty asm that "changes" jv and jf before each loop keeps the compiler
  // from holding 2 x J row masks in scalar registers across loops
#define SPTS_FRESH_ROWS() asm volatile("" : "+v"(jv), "+v"(jf))
  uint32_t kr[IPT];
  uint32_t k_or = 0u, k_and = 0xFFFFFFFFu;             // over the free rows
  {
    // every load is issued before any is used (the score/fusion choice is
    // made outside the row loop), so a lane's loads are in flight together;
    // kr holds the raw score bits until they become keys
    if (!s_b) {
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const int i = base + 64 * j;
        kr[j] = i < n ? __float_as_uint(s_a[i]) : 0u;
      }
    } else {
      float xb[IPT];
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const int i = base + 64 * j;
        kr[j] = i < n ? __float_as_uint(s_a[i]) : 0u;
        xb[j] = i < n ? s_b[i] : 0.f;
      }
      if (!mult) {
        float la = -INFINITY, lb = -INFINITY;
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
          const bool v = j < jv;
          la = fmaxf(la, v ? __uint_as_float(kr[j]) : -INFINITY);
          lb = fmaxf(lb, v ? xb[j] : -INFINITY);
        }
        block_max2(la, lb, red, ma, mb);
      }
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const float a = __uint_as_float(kr[j]);
        kr[j] = __float_as_uint(mult ? __fmul_rn(a, xb[j]) : fuse(a, xb[j], ma, mb, wa, wb));
      }
    }
    if (fused_out) {
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const int i = base + 64 * j;
        if (i < n) fused_out[i] = __uint_as_float(kr[j]);
      }
    }
    SPTS_FRESH_ROWS();
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const uint32_t key = j < jv ? order_key(__uint_as_float(kr[j])) : 0u;
      const bool fr = j < jf;
      k_or |= fr ? key : 0u;
      k_and &= fr ? key : 0xFFFFFFFFu;
      kr[j] = key;
    }
  }
  if (k >= n) return;

  auto key_at = [&](int j) -> uint32_t { return kr[j]; };

  const int kp = k - nf;            // rows to choose among the free ones
  uint32_t T = 0xFFFFFFFFu;         // no free row is selected when kp == 0 (no key is all ones)
  int need_eq = 0;
  if (kp > 0) {
    // bits shared by every free key need no radix pass
    k_or = wave_or(k_or);
    k_and = wave_and(k_and);
    if (lane == 0) { bits_sh[0][w] = k_or; bits_sh[1][w] = k_and; }
    __syncthreads();
    k_or = 0u; k_and = 0xFFFFFFFFu;
    for (int q = 0; q < NW; ++q) { k_or |= bits_sh[0][q]; k_and &= bits_sh[1][q]; }
    const uint32_t vary = k_or & ~k_and;
    int R = vary ? 32 - __clz(vary) : 0;          // bits below the common prefix
    uint32_t mask = R >= 32 ? 0u : ~((1u << R) - 1u);
    uint32_t prefix = k_and & mask;
    int rem = kp;
    // ---- first digit: B1 bits, one shared histogram (every free key carries the prefix)
    if (R > 0) {
      const int width = R < B1 ? R : B1;
      const int shift = R - width;
      const uint32_t dmask = (1u << width) - 1u;
      for (int i = tid; i < NB1; i += TPB) hist1[i] = 0;
      if (tid == 0) ccount = 0;
      __syncthreads();
      SPTS_FRESH_ROWS();
#pragma unroll UNROLL_J
      for (int j = 0; j < J; ++j)
        atomicAdd(&hist1[j < jf ? (int)((key_at(j) >> shift) & dmask) : NB1 + lane], 1);
      __syncthreads();
      if (w == 0) {
        int d, above, cnt;
        wave_find_digit<NB1>(hist1, rem, lane, d, above, cnt);
        if (lane == 0) { sel[0] = d; sel[1] = rem - above; sel[2] = cnt; }
      }
      __syncthreads();
      prefix |= (uint32_t)sel[0] << shift;
      rem = sel[1];
      mask |= dmask << shift;
      R = shift;
      const int c = sel[2];
      if (R > 0 && c <= CAP) {
        // ---- the c keys of that bin go to LDS (any order); one wave finishes them
        int mc = 0;
        SPTS_FRESH_ROWS();
#pragma unroll UNROLL_J
        for (int j = 0; j < J; ++j) mc += ((j < jf) & ((key_at(j) & mask) == prefix)) ? 1 : 0;
        const int incl_c = wave_incl_scan(mc);
        const int excl = incl_c - mc;
        const int tot = __builtin_amdgcn_readlane(incl_c, 63);
        int wb = 0;
        if (lane == 0 && tot > 0) wb = atomicAdd(&ccount, tot);
        int slot = __builtin_amdgcn_readfirstlane(wb) + excl;
        SPTS_FRESH_ROWS();
#pragma unroll UNROLL_J
        for (int j = 0; j < J; ++j) {
          const uint32_t key = key_at(j);
          const bool match = (j < jf) & ((key & mask) == prefix);
          pool[match ? slot : CAP + lane] = key;
          slot += match ? 1 : 0;
        }
        __syncthreads();
        if (w == 0) {
          // bits every candidate shares need no digit (all equal: done at once)
          uint32_t o = 0u, an = 0xFFFFFFFFu;
#pragma unroll 8
          for (int q = lane; q < c; q += 64) { o |= pool[q]; an &= pool[q]; }
          o = wave_or(o);
          an = wave_and(an);
          const uint32_t low = (1u << R) - 1u;
          const uint32_t var = (o & ~an) & low;
          const int Rn = var ? 32 - __clz(var) : 0;
          const uint32_t fixed = low & ~(Rn >= 32 ? 0u : ((1u << Rn) - 1u));
          prefix |= an & fixed;
          mask |= fixed;
          R = Rn;
          while (R > 0) {
            const int wd = R < 8 ? R : 8;
            const int sft = R - wd;
            const uint32_t dm = (1u << wd) - 1u;
            for (int q = lane; q < 256; q += 64) h8[q] = 0;
#pragma unroll 8
            for (int q = lane; q < c; q += 64) {
              const uint32_t key = pool[q];
              atomicAdd(&h8[(key & mask) == prefix ? (int)((key >> sft) & dm) : 256 + lane], 1);
            }
            int d, above, cnt;
            wave_find_digit<256>(h8, rem, lane, d, above, cnt);
            prefix |= (uint32_t)d << sft;
            rem -= above;
            mask |= dm << sft;
            R = sft;
          }
          if (lane == 0) { sel[0] = (int)prefix; sel[1] = rem; }
        }
        __syncthreads();
        prefix = (uint32_t)sel[0];
        rem = sel[1];
        R = 0;
      }
    }
    // ---- a large bin (many equal keys): 8-bit digits over the whole workgroup
    while (R > 0) {
      const int width = R < 8 ? R : 8;
      const int shift = R - width;
      const uint32_t dmask = (1u << width) - 1u;
      for (int i = tid; i < NW * 320; i += TPB) (&hist[0][0])[i] = 0;
      __syncthreads();
      SPTS_FRESH_ROWS();
#pragma unroll UNROLL_J
      for (int j = 0; j < J; ++j) {
        const uint32_t key = key_at(j);
        atomicAdd(&hist[w][((j < jf) & ((key & mask) == prefix)) ? (int)((key >> shift) & dmask) : 256 + lane], 1);
      }
      __syncthreads();
      if (tid < 256) {
        int t = 0;
        for (int q = 0; q < NW; ++q) t += hist[q][tid];
        tot_hist[tid] = t;
      }
      __syncthreads();
      if (w == 0) {
        int d, above, cnt;
        wave_find_digit<256>(tot_hist, rem, lane, d, above, cnt);
        if (lane == 0) { sel[0] = d; sel[1] = rem - above; }
      }
      __syncthreads();
      prefix |= (uint32_t)sel[0] << shift;
      rem = sel[1];
      mask |= dmask << shift;
      R = shift;
      __syncthreads();
    }
    T = prefix;
    need_eq = rem;
  }

  // ---- compaction in index order.  Per wave: rows above T (and forced rows)
  // and rows equal to T; then each wave knows how many equal rows precede it
  // and so how many of its own equal rows it takes, and where its output starts.
  int n_gt = 0, n_eq = 0;
  SPTS_FRESH_ROWS();
#pragma unroll UNROLL_J
  for (int j = 0; j < J; ++j) {
    const uint32_t key = key_at(j);
    const bool forced = (j >= jf) & (j < jv);
    const bool free_row = j < jf;
    n_gt += (forced | (free_row & (key > T))) ? 1 : 0;
    n_eq += (free_row & (key == T)) ? 1 : 0;
  }
  n_gt = wave_sum_int(n_gt);
  n_eq = wave_sum_int(n_eq);
  if (lane == 0) { cnt_sh[0][w] = n_gt; cnt_sh[1][w] = n_eq; }
  __syncthreads();
  // wave q's output starts after the rows taken by waves 0..q-1: lanes 0..NW-1
  // hold the per-wave counts and scan them
  const int g_q = lane < NW ? cnt_sh[0][lane] : 0;
  const int e_q = lane < NW ? cnt_sh[1][lane] : 0;
  const int e_excl = wave_incl_scan(e_q) - e_q;               // equal rows in earlier waves
  const int t_q = g_q + min(max(need_eq - e_excl, 0), e_q);    // rows wave q takes
  const int t_excl = wave_incl_scan(t_q) - t_q;
  int eq_before = __builtin_amdgcn_readlane(e_excl, w), out = __builtin_amdgcn_readlane(t_excl, w);
  const int e_total = __builtin_amdgcn_readlane(e_excl + e_q, NW - 1);
  if (need_eq >= e_total) {
    // every row equal to T is taken (no tie at the threshold): take key >= T
    SPTS_FRESH_ROWS();
#pragma unroll UNROLL_J
    for (int j = 0; j < J; ++j) {
      const int i = base + 64 * j;
      const uint32_t key = key_at(j);
      const bool take = (j >= jf) & (j < jv) | (j < jf) & (key >= T);
      const uint64_t tm = __ballot(take);
      const int pos = out + lanes_below(tm);
      if (take & (pos < k)) idx[pos] = i;  // exactly k are taken; the bound only guards memory
      out += __popcll(tm);
    }
    return;
  }
  // a tie at the threshold: the lowest-index need_eq of the rows equal to T
  SPTS_FRESH_ROWS();
#pragma unroll UNROLL_J
  for (int j = 0; j < J; ++j) {
    const int i = base + 64 * j;
    const uint32_t key = key_at(j);
    const bool free_row = j < jf;
    const bool eq = free_row & (key == T);
    const uint64_t eqm = __ballot(eq);
    const bool take = (j >= jf) & (j < jv) | free_row & (key > T) |
                      eq & (eq_before + lanes_below(eqm) < need_eq);
    const uint64_t tm = __ballot(take);
    const int pos = out + lanes_below(tm);
    if (take & (pos < k)) idx[pos] = i;    // exactly k are taken; the bound only guards memory
    out += __popcll(tm);
    eq_before += __popcll(eqm);
  }
#undef SPTS_FRESH_ROWS
}

// ------------------------------------------- many-workgroup select (n > 32K)
// Above 32K scores a single workgroup cannot keep the keys in registers, so
// the selection spreads over the chip.  Three radix digits (bits 31..21,
// 20..10, 9..0) are counted by all workgroups into global histograms (integer
// atomics: exact), each pass recovering the earlier digits from the earlier
// histograms itself (no separate launch per digit); a count pass fixes the
// threshold key T and how many rows equal to T to take and counts each
// workgroup's contiguous row range, a one-workgroup scan turns the counts
// into output offsets, and a write pass emits the indices in index order.
// Same selection as topk_kernel: forced rows, free rows above T, and the
// lowest-index need_eq free rows equal to T.  A fused score is formed in every
// pass with the same fp32 operations as topk_kernel; MaxNorm-Add needs the two
// maxima first, one more pass (atomicMax over order keys, so NaN is skipped
// as there).
constexpr int MT = 256;                       // threads per workgroup of these passes
constexpr int MG = 256;                       // most workgroups of the count / write passes
constexpr int MB = 2048;                      // bins of the 11-bit digits (the last digit uses 1024)
// workspace ints: hist[3][MB] | st[4] (T, need_eq, max key of s_a, of s_b) | counts[2 MG] | offs[2 MG]
constexpr int M_ST = 3 * MB, M_CNT = M_ST + 4, M_OFF = M_CNT + 2 * MG;

__device__ __forceinline__ int digit_shift(int p) { return p == 0 ? 21 : p == 1 ? 10 : 0; }
__device__ __forceinline__ int digit_bins(int p) { return p == 2 ? 1024 : 2048; }

// inclusive scan of one int per thread over the 256-thread workgroup
__device__ __forceinline__ int block_incl_scan(int v, int* sh) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int incl = wave_incl_scan(v);
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int q = 0; q < MT / 64; ++q) before += q < w ? sh[q] : 0;
  __syncthreads();
  return before + incl;
}

// The digits of passes 0 .. np-1 from their histograms: the bin holding the
// rem-th largest counted key, bins scanned from the top.  Every thread of the
// workgroup returns the same prefix, mask and remaining rank.
__device__ void find_digits(const int* __restrict__ hist, int np, uint32_t& prefix, uint32_t& mask, int& rem,
                            int* sh) {
  const int t = threadIdx.x;
  for (int p = 0; p < np; ++p) {
    const int nb = digit_bins(p), per = nb / MT;
    const int* h = hist + p * MB;
    int c[8];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      c[q] = q < per ? h[nb - 1 - (t * per + min(q, per - 1))] : 0;   // this thread's bins, descending
      sum += c[q];
    }
    const int incl = block_incl_scan(sum, sh);
    const int excl = incl - sum;
    if (excl < rem && rem <= incl) {                      // exactly one thread holds the crossing
      int acc = excl, d = -1;                             // acc: keys in bins above d
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (d < 0 && q < per) {
          if (rem <= acc + c[q]) d = nb - 1 - (t * per + q);
          else acc += c[q];
        }
      }
      sh[MT / 64] = d;
      sh[MT / 64 + 1] = rem - acc;
    }
    __syncthreads();
    const int d = sh[MT / 64];
    rem = sh[MT / 64 + 1];
    __syncthreads();
    const int sft = digit_shift(p);
    prefix |= (uint32_t)d << sft;
    mask |= (uint32_t)(nb - 1) << sft;
  }
}

// the scores being ranked: s_a alone, or s_a fused with s_b
struct MScores {
  const float* a;
  const float* b;       // nullptr: plain
  float wa, wb;
  int mult;
};

// inverse of order_key (a NaN never reaches it: its key 0 is below every init)
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float mscore(const MScores& sc, int i, float ma, float mb) {
  const float a = sc.a[i];
  if (!sc.b) return a;
  const float b = sc.b[i];
  return sc.mult ? __fmul_rn(a, b) : fuse(a, b, ma, mb, sc.wa, sc.wb);
}

// the maxima of MaxNorm-Add (st[2], st[3] hold their order keys)
__device__ __forceinline__ void mscore_maxima(const MScores& sc, const int* __restrict__ ws, float& ma,
                                              float& mb) {
  ma = mb = 0.f;
  if (sc.b && !sc.mult) {
    ma = key_float((uint32_t)ws[M_ST + 2]);
    mb = key_float((uint32_t)ws[M_ST + 3]);
  }
}

__global__ __launch_bounds__(MT) void mtopk_init_kernel(int* __restrict__ ws) {
  for (int i = threadIdx.x; i < 3 * MB; i += MT) ws[i] = 0;
  if (threadIdx.x < 2) ws[M_ST + 2 + threadIdx.x] = (int)order_key(-INFINITY);
}

// maxima of s_a and s_b over all rows, NaN skipped (fmaxf), as order keys
__global__ __launch_bounds__(MT) void mtopk_max_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                       int n, int* __restrict__ ws) {
  float la = -INFINITY, lb = -INFINITY;
  for (int i = blockIdx.x * MT + threadIdx.x; i < n; i += gridDim.x * MT) {
    la = fmaxf(la, a[i]);
    lb = fmaxf(lb, b[i]);
  }
  la = wave_max(la);
  lb = wave_max(lb);
  if ((threadIdx.x & 63) == 0) {
    atomicMax(reinterpret_cast<unsigned int*>(ws + M_ST + 2), order_key(la));
    atomicMax(reinterpret_cast<unsigned int*>(ws + M_ST + 3), order_key(lb));
  }
}

// pass P: histogram of digit P over the free keys that carry the earlier digits
template <int P>
__global__ __launch_bounds__(MT) void mtopk_hist_kernel(MScores sc, int nfree, int kp, int* __restrict__ ws) {
  __shared__ int lh[MB];
  __shared__ int sh[8];
  uint32_t prefix = 0u, mask = 0u;
  int rem = kp;
  float ma, mb;
  mscore_maxima(sc, ws, ma, mb);
  find_digits(ws, P, prefix, mask, rem, sh);
  const int nb = digit_bins(P), sft = digit_shift(P);
  for (int i = threadIdx.x; i < nb; i += MT) lh[i] = 0;
  __syncthreads();
  for (int i = blockIdx.x * MT + threadIdx.x; i < nfree; i += gridDim.x * MT) {
    const uint32_t key = order_key(mscore(sc, i, ma, mb));
    if ((key & mask) == prefix) atomicAdd(&lh[(key >> sft) & (uint32_t)(nb - 1)], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += MT)
    if (lh[i]) atomicAdd(&ws[P * MB + i], lh[i]);
}

// threshold T and need_eq from the three histograms; per workgroup range
// [b R, (b + 1) R): rows taken for sure (forced, or free above T) and free rows equal to T
__global__ __launch_bounds__(MT) void mtopk_count_kernel(MScores sc, int n, int nfree, int kp, int R,
                                                         float* __restrict__ fused_out, int* __restrict__ ws) {
  __shared__ int sh[8];
  float ma, mb;
  mscore_maxima(sc, ws, ma, mb);
  uint32_t T = 0xFFFFFFFFu;                                // kp == 0: no free row is taken
  int need_eq = 0;
  if (kp > 0) {
    uint32_t mask = 0u;
    T = 0u;
    need_eq = kp;
    find_digits(ws, 3, T, mask, need_eq, sh);
  }
  const int b0 = blockIdx.x * R, b1 = min(n, b0 + R);
  int g = 0, e = 0;
  for (int i = b0 + threadIdx.x; i < b1; i += MT) {
    const float x = mscore(sc, i, ma, mb);
    if (fused_out) fused_out[i] = x;
    const uint32_t key = order_key(x);
    const bool free_row = i < nfree;
    g += (!free_row | (key > T)) ? 1 : 0;
    e += (free_row & (key == T)) ? 1 : 0;
  }
  g = block_incl_scan(g, sh);                               // thread MT-1 holds the totals
  e = block_incl_scan(e, sh);
  if (threadIdx.x == MT - 1) {
    ws[M_CNT + 2 * blockIdx.x] = g;
    ws[M_CNT + 2 * blockIdx.x + 1] = e;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ws[M_ST] = (int)T;
    ws[M_ST + 1] = need_eq;
  }
}

// output offset and equal rows before each workgroup's range (one workgroup, G <= MG)
__global__ __launch_bounds__(MT) void mtopk_scan_kernel(int G, int* __restrict__ ws) {
  __shared__ int sh[8];
  const int t = threadIdx.x;
  const int need_eq = ws[M_ST + 1];
  const int g = t < G ? ws[M_CNT + 2 * t] : 0;
  const int e = t < G ? ws[M_CNT + 2 * t + 1] : 0;
  const int e_excl = block_incl_scan(e, sh) - e;
  const int take = g + min(max(need_eq - e_excl, 0), e);
  const int t_excl = block_incl_scan(take, sh) - take;
  if (t < G) {
    ws[M_OFF + 2 * t] = t_excl;
    ws[M_OFF + 2 * t + 1] = e_excl;
  }
}

// exclusive count of `flag` over the workgroup's threads in thread order, and the total
__device__ __forceinline__ int block_excl_count(bool flag, int* sh, int& total) {
  const int w = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  if ((threadIdx.x & 63) == 0) sh[w] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int q = 0; q < MT / 64; ++q) {
    before += q < w ? sh[q] : 0;
    total += sh[q];
  }
  __syncthreads();
  return before + lanes_below(m);
}

__global__ __launch_bounds__(MT) void mtopk_write_kernel(MScores sc, int n, int nfree, int k, int R,
                                                         const int* __restrict__ ws, int32_t* __restrict__ idx) {
  __shared__ int sh[8];
  float ma, mb;
  mscore_maxima(sc, ws, ma, mb);
  const uint32_t T = (uint32_t)ws[M_ST];
  const int need_eq = ws[M_ST + 1];
  int out = ws[M_OFF + 2 * blockIdx.x], eq_before = ws[M_OFF + 2 * blockIdx.x + 1];
  const int b0 = blockIdx.x * R, b1 = min(n, b0 + R);
  for (int c0 = b0; c0 < b1; c0 += MT) {                    // uniform over the workgroup
    const int i = c0 + threadIdx.x;
    const bool valid = i < b1;
    const uint32_t key = valid ? order_key(mscore(sc, i, ma, mb)) : 0u;
    const bool free_row = valid & (i < nfree);
    const bool eq = free_row & (key == T);
    int n_eq, n_take;
    const int er = eq_before + block_excl_count(eq, sh, n_eq);
    const bool take = (valid & !free_row) | (free_row & (key > T)) | (eq & (er < need_eq));
    const int pos = out + block_excl_count(take, sh, n_take);
    if (take & (pos < k)) idx[pos] = i;                     // exactly k are taken; the bound only guards memory
    out += n_take;
    eq_before += n_eq;
  }
}

__global__ void iota_kernel(int n, int32_t* __restrict__ idx) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) idx[i] = i;
}

}  // namespace

hipError_t launch_topk_batched(const float* s, long s_stride, int batch, int n, int k, int n_forced, int32_t* idx,
                               long idx_stride, hipStream_t st) {
  if (batch == 0) return hipSuccess;
  if (n <= TPB * 8)
    hipLaunchKernelGGL(topk_kernel<8>, dim3(batch), dim3(TPB), 0, st, s, nullptr, 0.f, 0.f, 0, n, k, n_forced, idx,
                       nullptr, s_stride, idx_stride);
  else
    hipLaunchKernelGGL(topk_kernel<32>, dim3(batch), dim3(TPB), 0, st, s, nullptr, 0.f, 0.f, 0, n, k, n_forced, idx,
                       nullptr, s_stride, idx_stride);
  return hipGetLastError();
}

size_t topk_workspace(int n) { return (((size_t)n * 4) + 255) & ~(size_t)255; }

// ---------------------------------------------------- allocation-free top-k
// Workspace of launch_topk_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends (a selection above 32K scores keeps its
// histograms and counters there, about 29 KiB; up to 32K none is used).  Its
// host-side name is not a device address; host code uses only the address
// hipGetSymbolAddress gives for the current device, resolved once per
// device.  Every call on one GPU shares it (the histograms are cleared by the
// call's own first kernel, every other slot is written before it is read),
// so calls that overlap on one GPU race.
static __device__ __align__(256) uint32_t scratch[kTopkNoallocMaxN];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
uint32_t* scratch_ptr[kMaxDevices];
}  // namespace

hipError_t launch_topk_noalloc(const float* s_a, const float* s_b, float w_a, float w_b, bool multiply, int n,
                               int k, int n_forced, int32_t* idx, float* fused_out, hipStream_t s) {
  if (n > kTopkNoallocMaxN) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint32_t* keys;
  {
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      scratch_ptr[dev] = reinterpret_cast<uint32_t*>(p);
    }
    keys = scratch_ptr[dev];
  }
  return launch_topk(s_a, s_b, w_a, w_b, multiply, n, k, n_forced, idx, fused_out, keys, s);
}

// selection over n > 32768 scores on many workgroups (ws: the call's
// workspace, at least topk_workspace(n) bytes, of which it uses about 30 KiB)
static hipError_t launch_topk_many(const float* s_a, const float* s_b, float w_a, float w_b, int mult, int n,
                                   int k, int n_forced, int32_t* idx, float* fused_out, int* ws, hipStream_t s) {
  const MScores sc{s_a, s_b, w_a, w_b, mult};
  if (k >= n && !(fused_out && s_b)) {
    hipLaunchKernelGGL(iota_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0, s, n, idx);
    return hipGetLastError();
  }
  const int nfree = n - n_forced, kp = k - n_forced;
  const int hist_blocks = std::min(1024, std::max(1, (nfree + 4 * MT - 1) / (4 * MT)));
  // contiguous row ranges of whole 256-row chunks, at most MG of them
  const int R = (((n + MG - 1) / MG) + MT - 1) / MT * MT;
  const int G = (n + R - 1) / R;
  hipLaunchKernelGGL(mtopk_init_kernel, dim3(1), dim3(MT), 0, s, ws);
  if (s_b && !mult)
    hipLaunchKernelGGL(mtopk_max_kernel, dim3(std::min(1024, (n + 4 * MT - 1) / (4 * MT))), dim3(MT), 0, s, s_a,
                       s_b, n, ws);
  if (k >= n) {
    // every row is taken; the fused scores are still written
    hipLaunchKernelGGL(mtopk_count_kernel, dim3(G), dim3(MT), 0, s, sc, n, nfree, 0, R, fused_out, ws);
    hipLaunchKernelGGL(iota_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0, s, n, idx);
    return hipGetLastError();
  }
  if (kp > 0) {
    hipLaunchKernelGGL(mtopk_hist_kernel<0>, dim3(hist_blocks), dim3(MT), 0, s, sc, nfree, kp, ws);
    hipLaunchKernelGGL(mtopk_hist_kernel<1>, dim3(hist_blocks), dim3(MT), 0, s, sc, nfree, kp, ws);
    hipLaunchKernelGGL(mtopk_hist_kernel<2>, dim3(hist_blocks), dim3(MT), 0, s, sc, nfree, kp, ws);
  }
  hipLaunchKernelGGL(mtopk_count_kernel, dim3(G), dim3(MT), 0, s, sc, n, nfree, kp, R, fused_out, ws);
  hipLaunchKernelGGL(mtopk_scan_kernel, dim3(1), dim3(MT), 0, s, G, ws);
  hipLaunchKernelGGL(mtopk_write_kernel, dim3(G), dim3(MT), 0, s, sc, n, nfree, k, R, ws, idx);
  return hipGetLastError();
}

hipError_t launch_topk(const float* s_a, const float* s_b, float w_a, float w_b, bool multiply, int n,
                       int k, int n_forced, int32_t* idx, float* fused_out, void* ws, hipStream_t s) {
  const int mult = multiply ? 1 : 0;
  // The fewest rows per lane that hold n: wave w owns rows [64 IPT w, 64 IPT (w + 1)),
  // so a larger IPT than needed leaves waves idle while the busy lanes walk
  // IPT keys in every pass (11,469 scores: 12 per lane on 15 waves instead of
  // 32 on 6).
  const auto go = [&](auto ipt) {
    hipLaunchKernelGGL(topk_kernel<decltype(ipt)::value>, dim3(1), dim3(TPB), 0, s, s_a, s_b, w_a, w_b, mult, n, k,
                       n_forced, idx, fused_out, 0L, 0L);
  };
  if (n <= TPB * 8) go(std::integral_constant<int, 8>{});
  else if (n <= TPB * 12) go(std::integral_constant<int, 12>{});
  else if (n <= TPB * 16) go(std::integral_constant<int, 16>{});
  else if (n <= TPB * 20) go(std::integral_constant<int, 20>{});
  else if (n <= TPB * 24) go(std::integral_constant<int, 24>{});
  else if (n <= TPB * 32) go(std::integral_constant<int, 32>{});
  else return launch_topk_many(s_a, s_b, w_a, w_b, mult, n, k, n_forced, idx, fused_out, reinterpret_cast<int*>(ws), s);
  return hipGetLastError();
}

}  // namespace spts
