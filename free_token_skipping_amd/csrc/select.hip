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
// reduction), so the first 8-bit digit already spreads the keys over many
// histogram bins instead of piling them onto one sign/exponent bin.
#include "common.hpp"
#include "kernels.hpp"

namespace spts {
namespace {

constexpr int TPB = 1024;
constexpr int NW = TPB / 64;

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

__device__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = -INFINITY;
  for (int i = 0; i < NW; ++i) r = fmaxf(r, sh[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
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
  __shared__ int hist[NW][256];          // one histogram per wave (less atomic contention)
  __shared__ int tot_hist[256];
  __shared__ float red[NW];
  __shared__ uint32_t bits_sh[2][NW];
  __shared__ int cnt_sh[2][NW];
  __shared__ int sel[2];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  s_a += (long)blockIdx.x * s_stride;    // batched rows (a single call: one workgroup, offsets 0)
  idx += (long)blockIdx.x * idx_stride;

  if (k >= n) {
    for (int i = tid; i < n; i += TPB) idx[i] = i;
    if (!(fused_out && s_b)) return;
  }

  float ma = 0.f, mb = 0.f;
  if (s_b && !mult) {
    float la = -INFINITY, lb = -INFINITY;
    for (int i = tid; i < n; i += TPB) { la = fmaxf(la, s_a[i]); lb = fmaxf(lb, s_b[i]); }
    ma = block_max(la, red);
    mb = block_max(lb, red);
  }
  constexpr int UNROLL_J = IPT > 0 ? IPT : 8;      // workspace keys: 8 loads in flight per lane
  const int nfree = n - nf;
  const int J = IPT > 0 ? IPT : (n + TPB - 1) / TPB;   // rows per lane (a constant if IPT > 0)
  const int base = w * J * 64 + lane;                  // row of (w, j, lane) = base + 64 j
  uint32_t kr[IPT > 0 ? IPT : 1];
  uint32_t k_or = 0u, k_and = 0xFFFFFFFFu;             // over the free rows
#pragma unroll UNROLL_J
  for (int j = 0; j < J; ++j) {
    const int i = base + 64 * j;
    uint32_t key = 0u;
    if (i < n) {
      const float x = !s_b ? s_a[i] : mult ? __fmul_rn(s_a[i], s_b[i]) : fuse(s_a[i], s_b[i], ma, mb, wa, wb);
      if (fused_out) fused_out[i] = x;
      key = order_key(x);
      if (i < nfree) { k_or |= key; k_and &= key; }
      if (IPT == 0) keys[i] = key;
    }
    if (IPT > 0) kr[IPT > 0 ? j : 0] = key;
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
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      k_or |= __shfl_xor(k_or, o);
      k_and &= __shfl_xor(k_and, o);
    }
    if (lane == 0) { bits_sh[0][w] = k_or; bits_sh[1][w] = k_and; }
    __syncthreads();
    k_or = 0u; k_and = 0xFFFFFFFFu;
    for (int q = 0; q < NW; ++q) { k_or |= bits_sh[0][q]; k_and &= bits_sh[1][q]; }
    const uint32_t vary = k_or & ~k_and;
    int R = vary ? 32 - __clz(vary) : 0;          // bits below the common prefix
    uint32_t mask = R >= 32 ? 0u : ~((1u << R) - 1u);
    uint32_t prefix = k_and & mask;
    int rem = kp;
    while (R > 0) {
      const int width = R < 8 ? R : 8;
      const int shift = R - width;
      const uint32_t dmask = (1u << width) - 1u;
      for (int i = tid; i < NW * 256; i += TPB) (&hist[0][0])[i] = 0;
      __syncthreads();
#pragma unroll UNROLL_J
      for (int j = 0; j < J; ++j) {
        const int i = base + 64 * j;
        const uint32_t key = key_at(j);
        if (i < nfree && (key & mask) == prefix) atomicAdd(&hist[w][(key >> shift) & dmask], 1);
      }
      __syncthreads();
      if (tid < 256) {
        int t = 0;
        for (int q = 0; q < NW; ++q) t += hist[q][tid];
        tot_hist[tid] = t;
      }
      __syncthreads();
      if (tid < 64) {
        // suffix sums over 256 bins, 4 bins per lane, highest digit first
        const int b0 = 255 - tid * 4;
        const int c0 = tot_hist[b0], c1 = tot_hist[b0 - 1], c2 = tot_hist[b0 - 2], c3 = tot_hist[b0 - 3];
        const int part = c0 + c1 + c2 + c3;
        int incl = part;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (tid >= o) incl += y;
        }
        const int excl = incl - part;   // keys with a larger digit than b0
        // the digit holding the rem-th largest lies in this lane's 4 bins iff excl < rem <= incl
        if (excl < rem && rem <= incl) {
          int above = excl, d = b0;
          const int cs[4] = {c0, c1, c2, c3};
          for (int q = 0; q < 4; ++q) {
            if (above + cs[q] >= rem) { d = b0 - q; break; }
            above += cs[q];
          }
          sel[0] = d;
          sel[1] = rem - above;
        }
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
#pragma unroll UNROLL_J
  for (int j = 0; j < J; ++j) {
    const int i = base + 64 * j;
    const uint32_t key = key_at(j);
    const bool forced = i >= nfree && i < n;
    const bool free_row = i < nfree;
    n_gt += __popcll(__ballot(forced || (free_row && key > T)));
    n_eq += __popcll(__ballot(free_row && key == T));
  }
  if (lane == 0) { cnt_sh[0][w] = n_gt; cnt_sh[1][w] = n_eq; }
  __syncthreads();
  int eq_before = 0, out = 0;
  for (int q = 0; q < w; ++q) {
    const int e = cnt_sh[1][q];
    out += cnt_sh[0][q] + min(max(need_eq - eq_before, 0), e);
    eq_before += e;
  }
#pragma unroll UNROLL_J
  for (int j = 0; j < J; ++j) {
    const int i = base + 64 * j;
    const uint32_t key = key_at(j);
    const bool free_row = i < nfree;
    const bool eq = free_row && key == T;
    const uint64_t eqm = __ballot(eq);
    const bool take = (i >= nfree && i < n) || (free_row && key > T) ||
                      (eq && eq_before + lanes_below(eqm) < need_eq);
    const uint64_t tm = __ballot(take);
    const int pos = out + lanes_below(tm);
    if (take && pos < k) idx[pos] = i;     // exactly k are taken; the bound only guards memory
    out += __popcll(tm);
    eq_before += __popcll(eqm);
  }
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
