// Decode-phase kernels (one new token per step), gfx950.
//
// After prefill every layer holds the K/V of its candidates; a decode step
// runs the new token through each layer: matrix-vector products against the
// weights (HBM-bound: every weight byte is read once per token) and one
// query against the layer's cached keys and values (HBM-bound on the cache).
//
// gemv_kernel: y[c] = sum_k x[k] W[c, k], bf16 in, fp32 accumulate.  One wave
// per output (a pair of outputs for RoPE, a gate/up pair for SwiGLU); its 64
// lanes stream the weight row 16 bytes at a time, 8 loads in flight per lane,
// against x staged once per workgroup in LDS.
//
// decode_attention: split over the cached keys.  Workgroup (chunk, KV head)
// scores its 256 keys against the G query heads of the group, keeps the
// chunk's softmax max, sum and unnormalised output per head; a combine kernel
// merges the chunks in chunk order (log-sum-exp), so the result does not
// depend on scheduling.
#include "common.hpp"
#include "kernels.hpp"

namespace spts {
namespace {

constexpr int GV_WAVES = 4;        // waves per workgroup
constexpr int GV_MAXK = 16384;     // largest inner dimension (x staged in LDS, 32 KiB)
constexpr int GV_BATCH = 8;        // 16-byte weight loads in flight per lane and row

// one weight row against x (in LDS): lane l takes bytes [16 l, 16 l + 16) of
// every 1 KiB step of the row
__device__ __forceinline__ float row_dot(const uint16_t* __restrict__ w, const uint16_t* xs, int K, int lane) {
  float acc = 0.f;
  for (int s0 = 0; s0 < K; s0 += GV_BATCH * 512) {
    u32x4 wr[GV_BATCH];
#pragma unroll
    for (int b = 0; b < GV_BATCH; ++b)
      if (s0 + b * 512 < K) wr[b] = ld16(w + s0 + b * 512 + lane * 8);
#pragma unroll
    for (int b = 0; b < GV_BATCH; ++b) {
      if (s0 + b * 512 >= K) break;
      const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + s0 + b * 512 + lane * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = __builtin_fmaf(lo_bf(xv[q]), lo_bf(wr[b][q]), acc);
        acc = __builtin_fmaf(hi_bf(xv[q]), hi_bf(wr[b][q]), acc);
      }
    }
  }
  return wave_sum(acc);
}

// EPI: 0 store, 1 RoPE (outputs c and c+64 of a 128-wide head), 2 SwiGLU
// (W = gate, W2 = up), 3 residual add (out = bf16(out + bf16(y))).
template <int EPI>
__global__ __launch_bounds__(GV_WAVES * 64) void gemv_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ w,
                                                             const uint16_t* __restrict__ w2, int K, int N,
                                                             uint16_t* __restrict__ out, int pos,
                                                             const float* __restrict__ table) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // K elements
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x * 8; i < K; i += GV_WAVES * 64 * 8) st16(xs + i, ld16(x + i));
  __syncthreads();
  const int wv = (int)blockIdx.x * GV_WAVES + (int)(threadIdx.x >> 6);   // this wave's work item
  if (EPI == 1) {
    // work item = (head, c < 64): outputs head*128 + c and head*128 + c + 64
    if (wv >= N / 2) return;
    const int head = wv / 64, c = wv % 64;
    const int o1 = head * 128 + c, o2 = o1 + 64;
    const float y1 = row_dot(w + (long)o1 * K, xs, K, lane);
    const float y2 = row_dot(w + (long)o2 * K, xs, K, lane);
    if (lane == 0) {
      const float cs = table[((long)pos * 64 + c) * 2], sn = table[((long)pos * 64 + c) * 2 + 1];
      out[o1] = f2bf(y1 * cs - y2 * sn);
      out[o2] = f2bf(y2 * cs + y1 * sn);
    }
    return;
  }
  if (wv >= N) return;
  const float y = row_dot(w + (long)wv * K, xs, K, lane);
  if (EPI == 2) {
    const float u = row_dot(w2 + (long)wv * K, xs, K, lane);
    if (lane == 0) out[wv] = f2bf((y / (1.0f + __expf(-y))) * u);
  } else if (EPI == 3) {
    if (lane == 0) out[wv] = f2bf(bf2f(out[wv]) + bf2f(f2bf(y)));
  } else {
    if (lane == 0) out[wv] = f2bf(y);
  }
}

template <int EPI>
hipError_t launch_gemv_k(const uint16_t* x, const uint16_t* w, const uint16_t* w2, int K, int N, uint16_t* out,
                         int pos, const float* table, hipStream_t s) {
  const int items = (EPI == 1) ? N / 2 : N;
  hipLaunchKernelGGL((gemv_kernel<EPI>), dim3((items + GV_WAVES - 1) / GV_WAVES), dim3(GV_WAVES * 64),
                     (size_t)K * sizeof(uint16_t), s, x, w, w2, K, N, out, pos, table);
  return hipGetLastError();
}

// ------------------------------------------------------------ decode attention
constexpr int DA_CHUNK = 256;      // cached keys per workgroup
constexpr int DA_G = 4;            // query heads per KV head handled by one workgroup
constexpr int DA_DH = 128;

// Partial softmax attention of the G query heads of KV head g over keys
// [c*256, c*256 + 256) of the cache.  Writes per head m (max, exp2 units),
// l (sum) and o[128] (unnormalised), into part[(c * Hq + h) * (DA_DH + 2)].
__global__ __launch_bounds__(256) void decode_attn_partial_kernel(const uint16_t* __restrict__ q,
                                                                  const uint16_t* __restrict__ kc,
                                                                  const uint16_t* __restrict__ vc, int L,
                                                                  int Hq, int Hkv, float sl2,
                                                                  float* __restrict__ part) {
  __shared__ float qs[DA_G][DA_DH];
  __shared__ float lg[DA_G][DA_CHUNK];
  __shared__ float ored[16][DA_G][DA_DH / 8][8];   // [key group][head][8-dim slice][element]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, g = blockIdx.y;
  const int h0 = g * DA_G;
  const int j0 = c * DA_CHUNK;
  const int nk = min(DA_CHUNK, L - j0);
  const long row = (long)Hkv * DA_DH;                 // elements between consecutive keys
  for (int i = tid; i < DA_G * DA_DH; i += 256) qs[i / DA_DH][i % DA_DH] = bf2f(q[(long)(h0 + i / DA_DH) * DA_DH + i % DA_DH]);
  __syncthreads();
  // logits: wave w takes keys w*64 .. w*64+63 of the chunk, 4 per instruction;
  // lane = (key within the 4) * 16 + 16-byte slice of the 256-byte row
  const int sub = lane >> 4, sl = lane & 15;
  u32x4 kr[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int j = wave * 64 + s * 4 + sub;
    if (j < nk) kr[s] = ld16(kc + (long)(j0 + j) * row + (long)g * DA_DH + sl * 8);
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int j = wave * 64 + s * 4 + sub;
    float d[DA_G];
#pragma unroll
    for (int h = 0; h < DA_G; ++h) {
      float a = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        a = __builtin_fmaf(lo_bf(kr[s][q4]), qs[h][sl * 8 + 2 * q4], a);
        a = __builtin_fmaf(hi_bf(kr[s][q4]), qs[h][sl * 8 + 2 * q4 + 1], a);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) a += __shfl_xor(a, o);   // sum over the 16 slices of the key
      d[h] = a;
    }
    if (sl == 0) {
#pragma unroll
      for (int h = 0; h < DA_G; ++h) lg[h][j] = (j < nk) ? d[h] * sl2 : -INFINITY;
    }
  }
  __syncthreads();
  // per head: max, exp2, sum (wave h reduces head h)
  float m = -INFINITY;
  for (int j = lane; j < DA_CHUNK; j += 64) m = fmaxf(m, lg[wave][j]);
  m = wave_max(m);
  float l = 0.f;
  for (int j = lane; j < DA_CHUNK; j += 64) {
    const float p = __builtin_amdgcn_exp2f(lg[wave][j] - m);
    lg[wave][j] = p;
    l += p;
  }
  l = wave_sum(l);
  float* ph = part + ((long)c * Hq + h0 + wave) * (DA_DH + 2);
  if (lane == 0) { ph[0] = m; ph[1] = l; }
  __syncthreads();
  // o[h][d] = sum_j p[h][j] v[j][d]: thread = (key group kg of 16, 8-dim slice ds);
  // a wave covers 4 keys' full rows per load
  const int kg = tid >> 4, ds = tid & 15;
  float acc[DA_G][8];
#pragma unroll
  for (int h = 0; h < DA_G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  for (int j = kg; j < nk; j += 16) {
    const u32x4 vr = ld16(vc + (long)(j0 + j) * row + (long)g * DA_DH + ds * 8);
#pragma unroll
    for (int h = 0; h < DA_G; ++h) {
      const float p = lg[h][j];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        acc[h][2 * q4] = __builtin_fmaf(p, lo_bf(vr[q4]), acc[h][2 * q4]);
        acc[h][2 * q4 + 1] = __builtin_fmaf(p, hi_bf(vr[q4]), acc[h][2 * q4 + 1]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < DA_G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) ored[kg][h][ds][e] = acc[h][e];
  __syncthreads();
  // fixed-order sum over the 16 key groups: thread = (head, dim)
  for (int i = tid; i < DA_G * DA_DH; i += 256) {
    const int h = i / DA_DH, dd = i % DA_DH;
    float t = 0.f;
    for (int k2 = 0; k2 < 16; ++k2) t += ored[k2][h][dd / 8][dd % 8];
    part[((long)c * Hq + h0 + h) * (DA_DH + 2) + 2 + dd] = t;
  }
}

// o[h][d] = sum_c 2^(m_c - M) o_c[d] / sum_c 2^(m_c - M) l_c, chunks in order
__global__ __launch_bounds__(DA_DH) void decode_attn_combine_kernel(const float* __restrict__ part, int nchunks,
                                                                    int Hq, uint16_t* __restrict__ o) {
  const int h = blockIdx.x, d = threadIdx.x;
  float M = -INFINITY;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, part[((long)c * Hq + h) * (DA_DH + 2)]);
  float num = 0.f, den = 0.f;
  for (int c = 0; c < nchunks; ++c) {
    const float* ph = part + ((long)c * Hq + h) * (DA_DH + 2);
    const float a = __builtin_amdgcn_exp2f(ph[0] - M);
    num = __builtin_fmaf(a, ph[2 + d], num);
    den = __builtin_fmaf(a, ph[1], den);
  }
  o[(long)h * DA_DH + d] = f2bf(num / den);
}

}  // namespace

size_t decode_attn_workspace(int L, int Hq) {
  const size_t nchunks = (size_t)(L + DA_CHUNK - 1) / DA_CHUNK;
  return nchunks * Hq * (DA_DH + 2) * sizeof(float);
}

hipError_t launch_decode_attn(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, int L, int Hq, int Hkv,
                              float scale, uint16_t* o, void* ws, hipStream_t s) {
  const int nchunks = (L + DA_CHUNK - 1) / DA_CHUNK;
  float* part = reinterpret_cast<float*>(ws);
  hipLaunchKernelGGL(decode_attn_partial_kernel, dim3(nchunks, Hkv), dim3(256), 0, s, q, kc, vc, L, Hq, Hkv,
                     scale * kLog2e, part);
  hipLaunchKernelGGL(decode_attn_combine_kernel, dim3(Hq), dim3(DA_DH), 0, s, part, nchunks, Hq, o);
  return hipGetLastError();
}

bool gemv_supported_k(int K) { return K > 0 && K % 512 == 0 && K <= GV_MAXK; }

hipError_t launch_gemv(const uint16_t* x, const uint16_t* w, const uint16_t* w2, int K, int N, uint16_t* out,
                       int epi, int pos, const float* table, hipStream_t s) {
  switch (epi) {
    case 0: return launch_gemv_k<0>(x, w, w2, K, N, out, pos, table, s);
    case 1: return launch_gemv_k<1>(x, w, w2, K, N, out, pos, table, s);
    case 2: return launch_gemv_k<2>(x, w, w2, K, N, out, pos, table, s);
    case 3: return launch_gemv_k<3>(x, w, w2, K, N, out, pos, table, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spts
