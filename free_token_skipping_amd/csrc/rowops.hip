// Row movement and small per-row kernels: gather / scatter / scatter-add of
// token rows (16-byte vector accesses on 8 KiB rows), RMSNorm, the RoPE
// cos/sin table and the LTP row-norm finish.  All are HBM-bound.
#include "common.hpp"
#include "kernels.hpp"

namespace spts {
namespace {

// One workgroup per (row, 4 KiB piece): unit = 16, 4 or 2 bytes.
template <int UNIT>
struct Unit;
template <> struct Unit<16> { typedef u32x4 T; };
template <> struct Unit<4> { typedef uint32_t T; };
template <> struct Unit<2> { typedef uint16_t T; };

template <int UNIT>
__global__ void gather_kernel(const char* __restrict__ src, const int32_t* __restrict__ idx, int k,
                              long units_per_row, char* __restrict__ dst) {
  typedef typename Unit<UNIT>::T T;
  const long total = (long)k * units_per_row;
  for (long u = (long)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (long)gridDim.x * blockDim.x) {
    const long row = u / units_per_row, col = u - row * units_per_row;
    const long s = (long)idx[row] * units_per_row + col;
    reinterpret_cast<T*>(dst)[u] = reinterpret_cast<const T*>(src)[s];
  }
}

template <int UNIT>
__global__ void scatter_kernel(const char* __restrict__ src, const int32_t* __restrict__ idx, int k,
                               long units_per_row, char* __restrict__ dst) {
  typedef typename Unit<UNIT>::T T;
  const long total = (long)k * units_per_row;
  for (long u = (long)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (long)gridDim.x * blockDim.x) {
    const long row = u / units_per_row, col = u - row * units_per_row;
    const long d = (long)idx[row] * units_per_row + col;
    reinterpret_cast<T*>(dst)[d] = reinterpret_cast<const T*>(src)[u];
  }
}

// bf16 rows, 8 elements per thread-step: dst[idx[i]] = bf16(dst + src).
__global__ void scatter_add_bf16_kernel(const uint16_t* __restrict__ src, const int32_t* __restrict__ idx,
                                        int k, int row_elems, uint16_t* __restrict__ dst) {
  const long vpr = row_elems / 8;
  const long total = (long)k * vpr;
  for (long u = (long)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (long)gridDim.x * blockDim.x) {
    const long row = u / vpr, col = u - row * vpr;
    const u32x4 a = ld16(src + u * 8);
    uint16_t* dp = dst + ((long)idx[row] * vpr + col) * 8;
    const u32x4 b = ld16(dp);
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      r[w] = pack2bf(lo_bf(a[w]) + lo_bf(b[w]), hi_bf(a[w]) + hi_bf(b[w]));
    st16(dp, r);
  }
}
__global__ void scatter_add_bf16_scalar_kernel(const uint16_t* __restrict__ src,
                                               const int32_t* __restrict__ idx, int k, int row_elems,
                                               uint16_t* __restrict__ dst) {
  const long total = (long)k * row_elems;
  for (long u = (long)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (long)gridDim.x * blockDim.x) {
    const long row = u / row_elems, col = u - row * row_elems;
    uint16_t* dp = dst + (long)idx[row] * row_elems + col;
    *dp = f2bf(bf2f(*dp) + bf2f(src[u]));
  }
}
template <typename T>
__global__ void scatter_add_kernel(const T* __restrict__ src, const int32_t* __restrict__ idx, int k,
                                   int row_elems, T* __restrict__ dst) {
  const long total = (long)k * row_elems;
  for (long u = (long)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (long)gridDim.x * blockDim.x) {
    const long row = u / row_elems, col = u - row * row_elems;
    dst[(long)idx[row] * row_elems + col] += src[u];
  }
}

// One workgroup per row; fp32 sum of squares, unit gain, bf16 output.  The
// first 8192 columns of the row stay in registers between the two passes
// (all their loads issued before the first is used); wider rows re-read the
// rest.  Thread t sums its 8-column groups t, t + 256, ... in that order.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int d, float eps,
                                                      uint16_t* __restrict__ out) {
  constexpr int R = 4;                       // 16-byte groups per thread held in registers
  __shared__ float red[4];
  const long row = blockIdx.x;
  const uint16_t* xr = x + row * d;
  u32x4 v[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int c = (threadIdx.x + i * 256) * 8;
    if (c < d) v[i] = ld16(xr + c);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if ((threadIdx.x + i * 256) * 8 < d) ss = sumsq8(v[i], ss);
  for (int c = (threadIdx.x + R * 256) * 8; c < d; c += 256 * 8) ss = sumsq8(ld16(xr + c), ss);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = rms_inv(red, d, eps);
  uint16_t* orow = out + row * d;
  auto scale = [&](const u32x4& u, int c) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = pack2bf(lo_bf(u[w]) * r, hi_bf(u[w]) * r);
    st16(orow + c, o);
  };
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int c = (threadIdx.x + i * 256) * 8;
    if (c < d) scale(v[i], c);
  }
  for (int c = (threadIdx.x + R * 256) * 8; c < d; c += 256 * 8) scale(ld16(xr + c), c);
}

// table[p, c] = (cos, sin)(p * theta^(-2c/dh)), angle in fp64.
__global__ void rope_table_kernel(int max_pos, int dh, double theta, float* __restrict__ table) {
  const int half = dh / 2;
  const long total = (long)max_pos * half;
  for (long u = (long)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += (long)gridDim.x * blockDim.x) {
    const long p = u / half;
    const int c = (int)(u - p * half);
    const double inv_freq = pow(theta, -2.0 * (double)c / (double)dh);
    const double ang = (double)p * inv_freq;
    table[2 * u] = (float)cos(ang);
    table[2 * u + 1] = (float)sin(ang);
  }
}

// out[i] = sqrt(sum_b partial[i, b]) in a fixed order.
__global__ void rowsum_sqrt_kernel(const float* __restrict__ partial, int n, int parts, float* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float t = 0.f;
  for (int b = 0; b < parts; ++b) t += partial[(long)i * parts + b];
  // a quadratic form with a positive semi-definite matrix can round to just
  // below zero when its value is ~0; NaN stays NaN
  out[i] = sqrtf(t < 0.f ? 0.f : t);
}

// G = V V^T for v_t = V^T [d, r]: workgroup (bx, by) computes the 16 x 16
// block G[16 by .., 16 bx ..], thread (ty, tx) one element.  The two 16-column
// slices of v_t pass through LDS 64 rows of k at a time (threads 0..127 load
// the row slice, 128..255 the column slice, 16 bytes each).  Products of bf16
// values are exact in fp64 and each element sums them in k order, so G is
// symmetric bit for bit.  Row i of gcat is [hi | hi | lo] with
// hi = bf16(G[i, :]) and lo = bf16(G[i, :] - hi).
__global__ __launch_bounds__(256) void ltp_gram_kernel(const uint16_t* __restrict__ v_t, int d, int r,
                                                       uint16_t* __restrict__ gcat) {
  __shared__ float sl[2][64][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int i0 = blockIdx.y * 16, j0 = blockIdx.x * 16;
  const int which = threadIdx.x >> 7;                       // 0: columns i0.., 1: columns j0..
  const int lr = (threadIdx.x & 127) >> 1, lc = (threadIdx.x & 1) * 8;
  const int c0 = which ? j0 : i0;
  double acc = 0.0;
  for (int k0 = 0; k0 < d; k0 += 64) {
    const int k = k0 + lr;
    u32x4 a = {0u, 0u, 0u, 0u};
    if (k < d) a = ld16(v_t + (long)k * r + c0 + lc);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sl[which][lr][lc + 2 * w] = lo_bf(a[w]);
      sl[which][lr][lc + 2 * w + 1] = hi_bf(a[w]);
    }
    __syncthreads();
    const int kn = min(64, d - k0);
    for (int kk = 0; kk < kn; ++kk) acc = fma((double)sl[0][kk][ty], (double)sl[1][kk][tx], acc);
    __syncthreads();
  }
  const int i = i0 + ty, j = j0 + tx;
  const uint16_t hi = f2bf((float)acc);
  const uint16_t lo = f2bf((float)(acc - (double)bf2f(hi)));
  uint16_t* row = gcat + (long)i * 3 * r;
  row[j] = hi;
  row[r + j] = hi;
  row[2 * r + j] = lo;
}

inline dim3 grid_for(long work, int tpb = 256) {
  long b = (work + tpb - 1) / tpb;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return dim3((unsigned)b);
}

}  // namespace

hipError_t launch_gather(const void* src, const int32_t* idx, int k, long row_bytes, void* dst, hipStream_t s) {
  if (k == 0) return hipSuccess;
  const char* sp = reinterpret_cast<const char*>(src);
  char* dp = reinterpret_cast<char*>(dst);
  if (row_bytes % 16 == 0)
    hipLaunchKernelGGL(gather_kernel<16>, grid_for(k * (row_bytes / 16)), dim3(256), 0, s, sp, idx, k, row_bytes / 16, dp);
  else if (row_bytes % 4 == 0)
    hipLaunchKernelGGL(gather_kernel<4>, grid_for(k * (row_bytes / 4)), dim3(256), 0, s, sp, idx, k, row_bytes / 4, dp);
  else
    hipLaunchKernelGGL(gather_kernel<2>, grid_for(k * (row_bytes / 2)), dim3(256), 0, s, sp, idx, k, row_bytes / 2, dp);
  return hipGetLastError();
}

hipError_t launch_scatter(const void* src, const int32_t* idx, int k, long row_bytes, void* dst, hipStream_t s) {
  if (k == 0) return hipSuccess;
  const char* sp = reinterpret_cast<const char*>(src);
  char* dp = reinterpret_cast<char*>(dst);
  if (row_bytes % 16 == 0)
    hipLaunchKernelGGL(scatter_kernel<16>, grid_for(k * (row_bytes / 16)), dim3(256), 0, s, sp, idx, k, row_bytes / 16, dp);
  else if (row_bytes % 4 == 0)
    hipLaunchKernelGGL(scatter_kernel<4>, grid_for(k * (row_bytes / 4)), dim3(256), 0, s, sp, idx, k, row_bytes / 4, dp);
  else
    hipLaunchKernelGGL(scatter_kernel<2>, grid_for(k * (row_bytes / 2)), dim3(256), 0, s, sp, idx, k, row_bytes / 2, dp);
  return hipGetLastError();
}

hipError_t launch_scatter_add_bf16(const uint16_t* src, const int32_t* idx, int k, int row_elems,
                                   uint16_t* dst, hipStream_t s) {
  if (k == 0) return hipSuccess;
  if (row_elems % 8 == 0)
    hipLaunchKernelGGL(scatter_add_bf16_kernel, grid_for((long)k * (row_elems / 8)), dim3(256), 0, s, src, idx, k, row_elems, dst);
  else
    hipLaunchKernelGGL(scatter_add_bf16_scalar_kernel, grid_for((long)k * row_elems), dim3(256), 0, s, src, idx, k, row_elems, dst);
  return hipGetLastError();
}
hipError_t launch_scatter_add_f32(const float* src, const int32_t* idx, int k, int row_elems, float* dst,
                                  hipStream_t s) {
  if (k == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_add_kernel<float>, grid_for((long)k * row_elems), dim3(256), 0, s, src, idx, k, row_elems, dst);
  return hipGetLastError();
}
hipError_t launch_scatter_add_i32(const int32_t* src, const int32_t* idx, int k, int row_elems, int32_t* dst,
                                  hipStream_t s) {
  if (k == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_add_kernel<int32_t>, grid_for((long)k * row_elems), dim3(256), 0, s, src, idx, k, row_elems, dst);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const uint16_t* x, int n, int d, float eps, uint16_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(n), dim3(256), 0, s, x, d, eps, out);
  return hipGetLastError();
}

hipError_t launch_rope_table(int max_pos, int dh, double theta, float* table, hipStream_t s) {
  hipLaunchKernelGGL(rope_table_kernel, grid_for((long)max_pos * (dh / 2)), dim3(256), 0, s, max_pos, dh, theta, table);
  return hipGetLastError();
}

hipError_t launch_rowsum_sqrt(const float* partial, int n, int parts, float* out, hipStream_t s) {
  hipLaunchKernelGGL(rowsum_sqrt_kernel, dim3((n + 255) / 256), dim3(256), 0, s, partial, n, parts, out);
  return hipGetLastError();
}

hipError_t launch_ltp_gram(const uint16_t* v_t, int d, int r, uint16_t* gcat, hipStream_t s) {
  hipLaunchKernelGGL(ltp_gram_kernel, dim3(r / 16, r / 16), dim3(256), 0, s, v_t, d, r, gcat);
  return hipGetLastError();
}

}  // namespace spts
