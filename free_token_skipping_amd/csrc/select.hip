// Top-k token selection with forced probe rows, gfx950.
//
// Scores (or the MaxNorm-Add or Multiply fusion of two scores) are mapped to unsigned
// keys whose integer order is the float order (NaN lowest, -0 == +0).  An
// MSB-first radix select over the non-forced rows finds the threshold key T
// of the (k - n_forced)-th largest and how many rows equal to T to take; a
// ballot compaction in index order then writes exactly k ascending indices:
// forced rows, rows above T, and the lowest-index rows equal to T.
//
// One 1024-thread workgroup does the whole selection: at 32K-128K scores the
// input is 128-512 KiB and the call is bound by latency, not bandwidth.  Wave
// w owns the contiguous rows [w*C, (w+1)*C) and its lanes walk them 64 at a
// time, so every load is one coalesced 256-byte access.  The radix passes
// skip the leading key bits that all free rows share (found by an OR/AND
// reduction).  The first digit is 11 bits wide and is counted in one shared
// 2048-bin histogram.  When the bin holding the threshold has at most CAP keys
// (the usual case), those keys are copied to LDS and a single wave finishes
// the remaining digits over them, with no workgroup barrier per digit; a
// larger bin (many equal scores) continues with 8-bit workgroup passes.
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

// IPT > 0: each lane keeps the keys of its IPT rows in registers across all
// passes (n <= 1024 * IPT).  IPT == 0: keys are re-read from the workspace.
template <int IPT>
__global__ __launch_bounds__(TPB) void topk_kernel(const float* __restrict__ s_a,
                                                   const float* __restrict__ s_b, float wa, float wb,
                                                   int mult, int n, int k, int nf, int32_t* __restrict__ idx,
                                                   float* __restrict__ fused_out,
                                                   uint32_t* __restrict__ keys, long s_stride,
                                                   long idx_stride) {
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

  float ma = 0.f, mb = 0.f;
  if (IPT == 0 && s_b && !mult) {           // (with IPT > 0 the maxima come from the loaded rows below)
    float la = -INFINITY, lb = -INFINITY;
    for (int i = tid; i < n; i += TPB) { la = fmaxf(la, s_a[i]); lb = fmaxf(lb, s_b[i]); }
    block_max2(la, lb, red, ma, mb);
  }
  constexpr int UNROLL_J = IPT > 0 ? IPT : 8;      // workspace keys: 8 loads in flight per lane
  const int nfree = n - nf;
  const int J = IPT > 0 ? IPT : (n + TPB - 1) / TPB;   // rows per lane (a constant if IPT > 0)
  const int base = w * J * 64 + lane;                  // row of (w, j, lane) = base + 64 j
  // a lane's rows base + 64 j are valid (< n) for j < jv and free (< nfree)
  // for j < jf; loops test j against these instead of keeping a mask per row
  int jv = n > base ? (n - base + 63) / 64 : 0;
  int jf = nfree > base ? (nfree - base + 63) / 64 : 0;
  // an empty asm that "changes" jv and jf before each loop keeps the compiler
  // from holding 2 x J row masks in scalar registers across loops
#define SPTS_FRESH_ROWS() asm volatile("" : "+v"(jv), "+v"(jf))
  uint32_t kr[IPT > 0 ? IPT : 1];
  uint32_t k_or = 0u, k_and = 0xFFFFFFFFu;             // over the free rows
  if (IPT > 0) {
    // every load is issued before any is used (the score/fusion choice is
    // made outside the row loop), so a lane's loads are in flight together;
    // kr holds the raw score bits until they become keys
    if (!s_b) {
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const int i = base + 64 * j;
        kr[IPT > 0 ? j : 0] = i < n ? __float_as_uint(s_a[i]) : 0u;
      }
    } else {
      float xb[IPT > 0 ? IPT : 1];
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const int i = base + 64 * j;
        kr[IPT > 0 ? j : 0] = i < n ? __float_as_uint(s_a[i]) : 0u;
        xb[j] = i < n ? s_b[i] : 0.f;
      }
      if (!mult) {
        float la = -INFINITY, lb = -INFINITY;
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
          const bool v = j < jv;
          la = fmaxf(la, v ? __uint_as_float(kr[IPT > 0 ? j : 0]) : -INFINITY);
          lb = fmaxf(lb, v ? xb[j] : -INFINITY);
        }
        block_max2(la, lb, red, ma, mb);
      }
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const float a = __uint_as_float(kr[IPT > 0 ? j : 0]);
        kr[IPT > 0 ? j : 0] = __float_as_uint(mult ? __fmul_rn(a, xb[j]) : fuse(a, xb[j], ma, mb, wa, wb));
      }
    }
    if (fused_out) {
#pragma unroll
      for (int j = 0; j < IPT; ++j) {
        const int i = base + 64 * j;
        if (i < n) fused_out[i] = __uint_as_float(kr[IPT > 0 ? j : 0]);
      }
    }
    SPTS_FRESH_ROWS();
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const uint32_t key = j < jv ? order_key(__uint_as_float(kr[IPT > 0 ? j : 0])) : 0u;
      const bool fr = j < jf;
      k_or |= fr ? key : 0u;
      k_and &= fr ? key : 0xFFFFFFFFu;
      kr[IPT > 0 ? j : 0] = key;
    }
  } else {
#pragma unroll UNROLL_J
    for (int j = 0; j < J; ++j) {
      const int i = base + 64 * j;
      if (i < n) {
        const float x = !s_b ? s_a[i] : mult ? __fmul_rn(s_a[i], s_b[i]) : fuse(s_a[i], s_b[i], ma, mb, wa, wb);
        if (fused_out) fused_out[i] = x;
        const uint32_t key = order_key(x);
        if (i < nfree) { k_or |= key; k_and &= key; }
        keys[i] = key;
      }
    }
  }
  if (k >= n) return;
  if (IPT == 0) __threadfence_block();

  auto key_at = [&](int j) -> uint32_t {
    if (IPT > 0) return kr[j];
    const int i = base + 64 * j;
    return i < n ? keys[i] : 0u;                // the workspace holds n keys
  };

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

}  // namespace

hipError_t launch_topk_batched(const float* s, long s_stride, int batch, int n, int k, int n_forced, int32_t* idx,
                               long idx_stride, hipStream_t st) {
  if (batch == 0) return hipSuccess;
  if (n <= TPB * 8)
    hipLaunchKernelGGL(topk_kernel<8>, dim3(batch), dim3(TPB), 0, st, s, nullptr, 0.f, 0.f, 0, n, k, n_forced, idx,
                       nullptr, nullptr, s_stride, idx_stride);
  else
    hipLaunchKernelGGL(topk_kernel<32>, dim3(batch), dim3(TPB), 0, st, s, nullptr, 0.f, 0.f, 0, n, k, n_forced, idx,
                       nullptr, nullptr, s_stride, idx_stride);
  return hipGetLastError();
}

size_t topk_workspace(int n) { return (((size_t)n * 4) + 255) & ~(size_t)255; }

hipError_t launch_topk(const float* s_a, const float* s_b, float w_a, float w_b, bool multiply, int n,
                       int k, int n_forced, int32_t* idx, float* fused_out, void* ws, hipStream_t s) {
  uint32_t* keys = reinterpret_cast<uint32_t*>(ws);
  const int mult = multiply ? 1 : 0;
  if (n <= TPB * 8)
    hipLaunchKernelGGL(topk_kernel<8>, dim3(1), dim3(TPB), 0, s, s_a, s_b, w_a, w_b, mult, n, k, n_forced, idx, fused_out, keys, 0L, 0L);
  else if (n <= TPB * 32)
    hipLaunchKernelGGL(topk_kernel<32>, dim3(1), dim3(TPB), 0, s, s_a, s_b, w_a, w_b, mult, n, k, n_forced, idx, fused_out, keys, 0L, 0L);
  else
    hipLaunchKernelGGL(topk_kernel<0>, dim3(1), dim3(TPB), 0, s, s_a, s_b, w_a, w_b, mult, n, k, n_forced, idx, fused_out, keys, 0L, 0L);
  return hipGetLastError();
}

}  // namespace spts
