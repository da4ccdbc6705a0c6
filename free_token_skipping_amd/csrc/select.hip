// Top-k token selection with forced probe rows, gfx950.
//
// Scores (or the MaxNorm-Add fusion of two scores) are mapped to unsigned
// keys whose integer order is the float order (NaN lowest, -0 == +0).  A
// 4-pass, 8-bit radix select over the non-forced rows finds the threshold
// key T of the (k - n_forced)-th largest and how many rows equal to T to
// take; a block-wide scan in index order then writes exactly k ascending
// indices: forced rows, rows above T, and the lowest-index rows equal to T.
// One 1024-thread workgroup does the whole selection: at 32K-128K scores the
// input is 128-512 KiB and the call is bound by latency, not bandwidth.
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

// MaxNorm-Add in fp32 with a fixed operation order (no contraction).
__device__ __forceinline__ float fuse(float a, float b, float ma, float mb, float wa, float wb) {
  const float ta = ma > 0.f ? __fmul_rn(wa, __fdiv_rn(a, ma)) : 0.f;
  const float tb = mb > 0.f ? __fmul_rn(wb, __fdiv_rn(b, mb)) : 0.f;
  return __fadd_rn(ta, tb);
}

// Exclusive scan over the block; returns this thread's prefix, *total = sum.
__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = lane < NW ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(t, o);
      if (lane >= o) t += y;
    }
    if (lane < NW) sh[NW + lane] = t;      // inclusive wave prefix
  }
  __syncthreads();
  const int wave_base = w ? sh[NW + w - 1] : 0;
  *total = sh[NW + NW - 1];
  __syncthreads();
  return wave_base + x - v;
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

// IPT > 0: each thread keeps the keys of its IPT contiguous rows in
// registers across all passes (n <= 1024 * IPT).  IPT == 0: keys are re-read
// from the workspace (any n).
template <int IPT>
__global__ __launch_bounds__(TPB) void topk_kernel(const float* __restrict__ s_a,
                                                   const float* __restrict__ s_b, float wa, float wb,
                                                   int n, int k, int nf, int32_t* __restrict__ idx,
                                                   float* __restrict__ fused_out,
                                                   uint32_t* __restrict__ keys) {
  __shared__ int hist[NW][256];          // one histogram per wave (less atomic contention)
  __shared__ int tot_hist[256];
  __shared__ int scan_sh[2 * NW];
  __shared__ float red[NW];
  __shared__ int sel[2];
  const int tid = threadIdx.x, w = tid >> 6;

  if (k >= n) {
    for (int i = tid; i < n; i += TPB) idx[i] = i;
    if (!(fused_out && s_b)) return;
  }

  float ma = 0.f, mb = 0.f;
  if (s_b) {
    float la = -INFINITY, lb = -INFINITY;
    for (int i = tid; i < n; i += TPB) { la = fmaxf(la, s_a[i]); lb = fmaxf(lb, s_b[i]); }
    ma = block_max(la, red);
    mb = block_max(lb, red);
  }
  const int per = IPT > 0 ? IPT : (n + TPB - 1) / TPB;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  uint32_t kr[IPT > 0 ? IPT : 1];
  if (IPT > 0) {
#pragma unroll
    for (int j = 0; j < (IPT > 0 ? IPT : 1); ++j) {
      const int i = lo + j;
      uint32_t key = 0u;
      if (i < hi) {
        const float x = s_b ? fuse(s_a[i], s_b[i], ma, mb, wa, wb) : s_a[i];
        if (fused_out) fused_out[i] = x;
        key = order_key(x);
      }
      kr[j] = key;
    }
  } else {
    for (int i = tid; i < n; i += TPB) {
      const float x = s_b ? fuse(s_a[i], s_b[i], ma, mb, wa, wb) : s_a[i];
      if (fused_out) fused_out[i] = x;
      keys[i] = order_key(x);
    }
    __threadfence_block();
  }
  if (k >= n) return;
  __syncthreads();

  auto key_at = [&](int j, int i) -> uint32_t { return IPT > 0 ? kr[j] : keys[i]; };

  const int nfree = n - nf;
  const int kp = k - nf;            // rows to choose among the free ones
  uint32_t T = 0xFFFFFFFFu;         // no free row is selected when kp == 0
  int need_eq = 0;
  if (kp > 0) {
    uint32_t prefix = 0, mask = 0;
    int rem = kp;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < NW * 256; i += TPB) (&hist[0][0])[i] = 0;
      __syncthreads();
      for (int j = 0, i = lo; i < min(hi, nfree); ++j, ++i) {
        const uint32_t key = key_at(j, i);
        if ((key & mask) == prefix) atomicAdd(&hist[w][(key >> shift) & 255], 1);
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
      const int d = sel[0];
      rem = sel[1];
      prefix |= (uint32_t)d << shift;
      mask |= 0xFFu << shift;
      __syncthreads();
    }
    T = prefix;
    need_eq = rem;
  }

  // compaction in index order over each thread's contiguous rows
  int n_eq = 0;
  for (int j = 0, i = lo; i < min(hi, nfree); ++j, ++i) n_eq += (key_at(j, i) == T);
  int tot;
  const int eq_rank = block_exclusive_scan(n_eq, scan_sh, &tot);
  int n_sel = 0;
  {
    int r = eq_rank;
    for (int j = 0, i = lo; i < hi; ++j, ++i) {
      bool take;
      if (i >= nfree) take = true;
      else {
        const uint32_t key = key_at(j, i);
        take = key > T || (key == T && r < need_eq);
        r += (key == T);
      }
      n_sel += take;
    }
  }
  int out = block_exclusive_scan(n_sel, scan_sh, &tot);
  {
    int r = eq_rank;
    for (int j = 0, i = lo; i < hi; ++j, ++i) {
      bool take;
      if (i >= nfree) take = true;
      else {
        const uint32_t key = key_at(j, i);
        take = key > T || (key == T && r < need_eq);
        r += (key == T);
      }
      if (take && out < k) idx[out++] = i;   // exactly k are taken; the bound only guards memory
    }
  }
}

}  // namespace

size_t topk_workspace(int n) { return (((size_t)n * 4) + 255) & ~(size_t)255; }

hipError_t launch_topk(const float* s_a, const float* s_b, float w_a, float w_b, int n, int k,
                       int n_forced, int32_t* idx, float* fused_out, void* ws, hipStream_t s) {
  uint32_t* keys = reinterpret_cast<uint32_t*>(ws);
  if (n <= TPB * 8)
    hipLaunchKernelGGL(topk_kernel<8>, dim3(1), dim3(TPB), 0, s, s_a, s_b, w_a, w_b, n, k, n_forced, idx, fused_out, keys);
  else if (n <= TPB * 32)
    hipLaunchKernelGGL(topk_kernel<32>, dim3(1), dim3(TPB), 0, s, s_a, s_b, w_a, w_b, n, k, n_forced, idx, fused_out, keys);
  else
    hipLaunchKernelGGL(topk_kernel<0>, dim3(1), dim3(TPB), 0, s, s_a, s_b, w_a, w_b, n, k, n_forced, idx, fused_out, keys);
  return hipGetLastError();
}

}  // namespace spts
