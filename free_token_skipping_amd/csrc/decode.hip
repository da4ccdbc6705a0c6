// Decode-phase kernels (one new token per step), gfx950.
//
// After prefill every layer holds the K/V of its candidates; a decode step
// runs the new token through each layer: matrix-vector products against the
// weights (HBM-bound: every weight byte is read once per token) and one
// query against the layer's cached keys and values (HBM-bound on the cache).
//
// gemv_kernel: y[c] = sum_k x[k] W[c, k], bf16 in, fp32 accumulate.  One wave
// per work item (one output; a pair of outputs c, c + 64 of a 128-wide head
// for RoPE; a gate/up pair for SwiGLU); its 64 lanes stream the weight rows
// 16 bytes at a time, 8 loads in flight per lane, against x staged once per
// workgroup in LDS.  With NORM the staged row is RMS-normalised first, with
// the same per-thread order as the RMSNorm kernel (identical bf16 values), so
// a layer needs no separate normalisation launch.  The QKV epilogue takes the
// three projections of a layer in one launch and writes K and V straight
// into the cache row of the new token.
//
// decode_attention: split over the cached keys.  Workgroup (chunk, KV head)
// scores its chunk of keys against the 4 query heads of the group and keeps
// the chunk's softmax max, sum and unnormalised output per head; a combine
// kernel merges the chunks (log-sum-exp) in a fixed order, so the result
// does not depend on scheduling.  A workgroup streams its chunk in 64-key
// tiles with the next tile's loads in flight and no barrier in the loop; the
// chunk is sized so that the grid has about two workgroups per compute unit.
#include "common.hpp"
#include "kernels.hpp"

namespace spts {
namespace {

constexpr int GV_WAVES = 4;        // waves per workgroup (256 threads, as the RMSNorm kernel)
constexpr int GV_MAXK = 16384;     // largest inner dimension (x staged in LDS, 32 KiB)
constexpr int GV_BATCH = 8;        // 16-byte weight loads in flight per lane and row

enum GemvEpi { GV_STORE = 0, GV_ROPE = 1, GV_SWIGLU = 2, GV_ADD = 3, GV_QKV = 4 };

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// c + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs (v_dot2c_f32_bf16):
// the bf16 products are exact in fp32, accumulated in fp32
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

struct GemvArgs {
  const uint16_t* x;
  const uint16_t* w[3];   // STORE/ROPE/ADD: w[0]; SWIGLU: gate, up; QKV: wq, wk, wv
  uint16_t* out[3];       // QKV: q, k row, v row
  int K;                  // inner dimension
  int N;                  // rows of w[0]
  int nkv;                // QKV: rows of wk and of wv
  int pos;                // RoPE position
  const float* table;     // RoPE table (QKV without RoPE: nullptr)
  float eps;              // NORM
};

// A weight row is read in batches of GV_BATCH 16-byte loads per lane (lane l
// takes bytes [16 l, 16 l + 16) of every 1 KiB step).  The first batch of a
// wave's rows is issued before x is staged; later batches are loaded while
// the previous one is consumed.
__device__ __forceinline__ void load_batch(const uint16_t* __restrict__ w, int s0, int K, int lane,
                                           u32x4 (&wr)[GV_BATCH]) {
#pragma unroll
  for (int b = 0; b < GV_BATCH; ++b)
    if (s0 + b * 512 < K) wr[b] = ld16(w + s0 + b * 512 + lane * 8);
}

// one weight row against x (in LDS), its first batch already in wr
__device__ __forceinline__ float row_dot(const uint16_t* __restrict__ w, const uint16_t* xs, int K, int lane,
                                         u32x4 (&wr)[GV_BATCH]) {
  float acc = 0.f;
  for (int s0 = 0; s0 < K; s0 += GV_BATCH * 512) {
    const bool more = s0 + GV_BATCH * 512 < K;
    u32x4 nx[GV_BATCH];
    if (more) load_batch(w, s0 + GV_BATCH * 512, K, lane, nx);
#pragma unroll
    for (int b = 0; b < GV_BATCH; ++b) {
      if (s0 + b * 512 >= K) break;
      const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + s0 + b * 512 + lane * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = dot2bf(xv[q], wr[b][q], acc);
    }
    if (more) {
#pragma unroll
      for (int b = 0; b < GV_BATCH; ++b) wr[b] = nx[b];
    }
  }
  return wave_sum(acc);
}

__device__ __forceinline__ void rope_pair(float y1, float y2, int pos, int c, const float* table, uint16_t* o1,
                                          uint16_t* o2) {
  const float cs = table[((long)pos * 64 + c) * 2], sn = table[((long)pos * 64 + c) * 2 + 1];
  *o1 = f2bf(y1 * cs - y2 * sn);
  *o2 = f2bf(y2 * cs + y1 * sn);
}

template <int EPI, bool NORM>
__global__ __launch_bounds__(GV_WAVES * 64) void gemv_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // K elements
  __shared__ float red[GV_WAVES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int K = a.K;
  const int wv = (int)blockIdx.x * GV_WAVES + (tid >> 6);   // this wave's work item
  constexpr bool kPair = (EPI == GV_ROPE || EPI == GV_QKV || EPI == GV_SWIGLU);
  // the work item's rows: ROPE/QKV item = (head, c < 64), outputs head*128 + c
  // and head*128 + c + 64; SWIGLU item c = gate row c and up row c
  const int items = (EPI == GV_QKV) ? (a.N + 2 * a.nkv) / 2 : (EPI == GV_ROPE) ? a.N / 2 : a.N;
  const bool valid = wv < items;
  int which = 0, o1 = wv, o2 = wv, c = 0;
  const uint16_t* r1 = nullptr;
  const uint16_t* r2 = nullptr;
  if (EPI == GV_ROPE || EPI == GV_QKV) {
    int head = wv / 64;
    c = wv % 64;
    if (EPI == GV_QKV) {
      const int hq = a.N / 128, hk = a.nkv / 128;
      if (head >= hq + hk) {
        which = 2;
        head -= hq + hk;
      } else if (head >= hq) {
        which = 1;
        head -= hq;
      }
    }
    o1 = head * 128 + c;
    o2 = o1 + 64;
    r1 = a.w[which] + (long)o1 * K;
    r2 = a.w[which] + (long)o2 * K;
  } else if (EPI == GV_SWIGLU) {
    r1 = a.w[0] + (long)wv * K;
    r2 = a.w[1] + (long)wv * K;
  } else {
    r1 = a.w[0] + (long)wv * K;
  }
  u32x4 w1[GV_BATCH], w2[GV_BATCH];
  if (valid) {
    load_batch(r1, 0, K, lane, w1);
    if (kPair) load_batch(r2, 0, K, lane, w2);
  }
  if (NORM) {
    float ss = 0.f;
    for (int i = tid * 8; i < K; i += GV_WAVES * 64 * 8) {
      const u32x4 v = ld16(a.x + i);
      ss = sumsq8(v, ss);
      st16(xs + i, v);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float r = rms_inv(red, K, a.eps);
    for (int i = tid * 8; i < K; i += GV_WAVES * 64 * 8) {   // the entries this thread staged
      const u32x4 v = *reinterpret_cast<const u32x4*>(xs + i);
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = pack2bf(lo_bf(v[w]) * r, hi_bf(v[w]) * r);
      st16(xs + i, o);
    }
  } else {
    for (int i = tid * 8; i < K; i += GV_WAVES * 64 * 8) st16(xs + i, ld16(a.x + i));
  }
  __syncthreads();
  if (!valid) return;
  const float y1 = row_dot(r1, xs, K, lane, w1);
  if (EPI == GV_ROPE || EPI == GV_QKV) {
    const float y2 = row_dot(r2, xs, K, lane, w2);
    uint16_t* out = a.out[which];
    if (lane == 0) {
      if (which < 2 && a.table != nullptr) {
        rope_pair(y1, y2, a.pos, c, a.table, out + o1, out + o2);
      } else {
        out[o1] = f2bf(y1);
        out[o2] = f2bf(y2);
      }
    }
  } else if (EPI == GV_SWIGLU) {
    const float u = row_dot(r2, xs, K, lane, w2);
    if (lane == 0) a.out[0][wv] = f2bf((y1 / (1.0f + __expf(-y1))) * u);
  } else if (EPI == GV_ADD) {
    if (lane == 0) a.out[0][wv] = f2bf(bf2f(a.out[0][wv]) + bf2f(f2bf(y1)));
  } else {
    if (lane == 0) a.out[0][wv] = f2bf(y1);
  }
}

template <int EPI, bool NORM>
hipError_t launch_gemv_k(const GemvArgs& a, hipStream_t s) {
  const int items = (EPI == GV_QKV) ? (a.N + 2 * a.nkv) / 2 : (EPI == GV_ROPE) ? a.N / 2 : a.N;
  hipLaunchKernelGGL((gemv_kernel<EPI, NORM>), dim3((items + GV_WAVES - 1) / GV_WAVES), dim3(GV_WAVES * 64),
                     (size_t)a.K * sizeof(uint16_t), s, a);
  return hipGetLastError();
}

template <bool NORM>
hipError_t launch_gemv_n(int epi, const GemvArgs& a, hipStream_t s) {
  switch (epi) {
    case GV_STORE: return launch_gemv_k<GV_STORE, NORM>(a, s);
    case GV_ROPE: return launch_gemv_k<GV_ROPE, NORM>(a, s);
    case GV_SWIGLU: return launch_gemv_k<GV_SWIGLU, NORM>(a, s);
    case GV_ADD: return launch_gemv_k<GV_ADD, NORM>(a, s);
    case GV_QKV: return launch_gemv_k<GV_QKV, NORM>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------ decode attention
constexpr int DA_G = 4;            // query heads per KV head handled by one workgroup
constexpr int DA_DH = 128;
constexpr int DA_MINCH = 64;       // smallest chunk: bounds the number of partials
constexpr int DA_PR = DA_DH + 4;   // floats per (chunk, head) partial: o[128], m, l, 2 pad (16-byte rows)

// DPP lane moves inside a row of 16 lanes (quad_perm, row_half_mirror,
// row_mirror); every lane of the row ends with the sum of the row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);    // lanes [1,0,3,2] of each quad
  x += dpp_mov<0x4E>(x);    // lanes [2,3,0,1] of each quad
  x += dpp_mov<0x141>(x);   // lane i <- 7 - i within each half row
  x += dpp_mov<0x140>(x);   // lane i <- 15 - i within the row
  return x;
}

// Partial softmax attention of the G query heads of KV head g over the keys
// [c*chunk, c*chunk + chunk) of the cache, streamed in tiles of 64 keys with
// the next tile's K and V rows in flight (registers, two sets).
//   lane layout, for K and for V alike: wave w takes keys 16 w .. 16 w + 15 of
//   a tile, 4 per load; lane = (key within the 4: its row of 16 lanes) * 16 +
//   16-byte slice of the 256-byte row (8 of the 128 dims).
// A key's logit is summed over its row of 16 lanes (DPP), so every lane that
// holds a slice of that key's V row also holds its logit: each lane keeps its
// own online softmax (running max, sum and output slice per head) over the
// keys its row sees, and the loop needs no barrier.  At the end the 16 row
// states of the workgroup are merged in a fixed order; the chunk's o[128]
// (unnormalised), m (max, exp2 units) and l (sum) per head go to
// part[(c * Hq + h) * DA_PR ...].
struct DecodeTile {
  u32x4 k[4], v[4];
};

__device__ __forceinline__ void load_tile(DecodeTile& t, const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ vb, long row, int jb, int nk, int sl) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int j = jb + s * 4;
    if (j < nk) {
      t.k[s] = ld16(kb + (long)j * row + sl * 8);
      t.v[s] = ld16(vb + (long)j * row + sl * 8);
    } else {
      t.k[s] = u32x4{0u, 0u, 0u, 0u};
      t.v[s] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__global__ __launch_bounds__(256) void decode_attn_partial_kernel(const uint16_t* __restrict__ q,
                                                                  const uint16_t* __restrict__ kc,
                                                                  const uint16_t* __restrict__ vc, int L,
                                                                  int chunk, int Hq, int Hkv, float sl2,
                                                                  float* __restrict__ part) {
  __shared__ float ms[16][DA_G];                 // [wave*4 + row][head]
  __shared__ float ls[16][DA_G];
  __shared__ float os[16][DA_G][DA_DH];          // 32 KiB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, g = blockIdx.y;
  const int h0 = g * DA_G;
  const int j0 = c * chunk;
  const int nk = min(chunk, L - j0);
  const int nt = (nk + 63) / 64;
  const long row = (long)Hkv * DA_DH;                 // elements between consecutive keys
  const int sub = lane >> 4, sl = lane & 15;
  const uint16_t* kb = kc + (long)j0 * row + (long)g * DA_DH;
  const uint16_t* vb = vc + (long)j0 * row + (long)g * DA_DH;
  const int jw = wave * 16 + sub;                     // this lane's first key of a tile; then + 4 s
  DecodeTile ta, tb;
  load_tile(ta, kb, vb, row, jw, nk, sl);
  u32x4 qv[DA_G];                                     // this lane's 8 dims of each head (bf16 pairs)
#pragma unroll
  for (int h = 0; h < DA_G; ++h) qv[h] = ld16(q + (long)(h0 + h) * DA_DH + sl * 8);
  float m[DA_G], l[DA_G], acc[DA_G][8];
#pragma unroll
  for (int h = 0; h < DA_G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  auto step = [&](const DecodeTile& t, int ti) {
    const int jb = ti * 64 + jw;
    float lg[4][DA_G];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bool ok = jb + s * 4 < nk;
#pragma unroll
      for (int h = 0; h < DA_G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) a = dot2bf(t.k[s][e], qv[h][e], a);
        a = row16_sum(a) * sl2;                           // logit in exp2 units
        lg[s][h] = ok ? a : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < DA_G; ++h) {
      const float mt = fmaxf(fmaxf(lg[0][h], lg[1][h]), fmaxf(lg[2][h], lg[3][h]));
      const float mn = fmaxf(m[h], mt);
      if (mn == -INFINITY) continue;                  // no key of this row seen yet (uniform in the row)
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);   // 0 while m[h] is -inf
      float p[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) p[s] = __builtin_amdgcn_exp2f(lg[s][h] - mn);
      l[h] = l[h] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[h][2 * e] = __builtin_fmaf(p[s], lo_bf(t.v[s][e]), acc[h][2 * e]);
          acc[h][2 * e + 1] = __builtin_fmaf(p[s], hi_bf(t.v[s][e]), acc[h][2 * e + 1]);
        }
      }
    }
  };

  for (int ti = 0; ti < nt; ti += 2) {
    if (ti + 1 < nt) load_tile(tb, kb, vb, row, (ti + 1) * 64 + jw, nk, sl);
    step(ta, ti);
    if (ti + 1 >= nt) break;
    if (ti + 2 < nt) load_tile(ta, kb, vb, row, (ti + 2) * 64 + jw, nk, sl);
    step(tb, ti + 1);
  }
  const int rs = wave * 4 + sub;                      // this lane's row state
  if (sl == 0) {
#pragma unroll
    for (int h = 0; h < DA_G; ++h) {
      ms[rs][h] = m[h];
      ls[rs][h] = l[h];
    }
  }
#pragma unroll
  for (int h = 0; h < DA_G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) os[rs][h][sl * 8 + e] = acc[h][e];
  __syncthreads();
  // merge the 16 row states in order: thread = (head, dim)
  for (int i = tid; i < DA_G * DA_DH; i += 256) {
    const int h = i / DA_DH, dd = i % DA_DH;
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) M = fmaxf(M, ms[r][h]);
    float o = 0.f, lt = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float a = ms[r][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[r][h] - M);
      o = __builtin_fmaf(a, os[r][h][dd], o);
      lt = __builtin_fmaf(a, ls[r][h], lt);
    }
    float* ph = part + ((long)c * Hq + h0 + h) * DA_PR;
    ph[dd] = o;
    if (dd == 0) {
      ph[DA_DH] = M;
      ph[DA_DH + 1] = lt;
    }
  }
}

// o[h][d] = sum_c 2^(m_c - M) o_c[d] / sum_c 2^(m_c - M) l_c.  Workgroup per
// head; thread (chunk group cg of 8, 4-dim quad dq) sums chunks cg, cg + 8, ...
// in order, then the 8 groups are added in order: a fixed summation tree.
__global__ __launch_bounds__(256) void decode_attn_combine_kernel(const float* __restrict__ part, int nchunks,
                                                                  int Hq, uint16_t* __restrict__ o) {
  __shared__ float wm[4];
  __shared__ float red[8][DA_DH + 1];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const long cs = (long)Hq * DA_PR;                 // floats between consecutive chunks of one head
  const float* ph = part + (long)h * DA_PR;
  float m = -INFINITY;
  for (int c = tid; c < nchunks; c += 256) m = fmaxf(m, ph[c * cs + DA_DH]);
  m = wave_max(m);
  if (lane == 0) wm[tid >> 6] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  const int cg = tid >> 5, dq = tid & 31;
  float n0 = 0.f, n1 = 0.f, n2 = 0.f, n3 = 0.f, den = 0.f;
#pragma unroll 4
  for (int c = cg; c < nchunks; c += 8) {
    const float* pc = ph + c * cs;
    const f32x4 v = *reinterpret_cast<const f32x4*>(pc + dq * 4);
    const float mc = pc[DA_DH], lc = pc[DA_DH + 1];
    const float a = __builtin_amdgcn_exp2f(mc - M);
    n0 = __builtin_fmaf(a, v[0], n0);
    n1 = __builtin_fmaf(a, v[1], n1);
    n2 = __builtin_fmaf(a, v[2], n2);
    n3 = __builtin_fmaf(a, v[3], n3);
    den = __builtin_fmaf(a, lc, den);
  }
  red[cg][dq * 4] = n0;
  red[cg][dq * 4 + 1] = n1;
  red[cg][dq * 4 + 2] = n2;
  red[cg][dq * 4 + 3] = n3;
  if (dq == 0) red[cg][DA_DH] = den;
  __syncthreads();
  if (tid < DA_DH) {
    float num = 0.f, dn = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      num += red[g][tid];
      dn += red[g][DA_DH];
    }
    o[(long)h * DA_DH + tid] = f2bf(num / dn);
  }
}

// keys per workgroup: a multiple of 64 giving about 512 workgroups over the
// KV heads (two resident per compute unit at this kernel's register use), so
// that every workgroup streams a few tiles
int decode_attn_chunk(int L, int Hkv) {
  const long tiles = ((long)L * Hkv + 512L * 64 - 1) / (512L * 64);
  return (int)(tiles < 1 ? 64 : tiles * 64);
}

size_t round_up256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

bool gemv_supported_k(int K) { return K > 0 && K % 512 == 0 && K <= GV_MAXK; }

hipError_t launch_gemv(const uint16_t* x, const uint16_t* w, const uint16_t* w2, int K, int N, uint16_t* out,
                       int epi, int pos, const float* table, hipStream_t s) {
  if (epi < GV_STORE || epi > GV_ADD) return hipErrorInvalidValue;
  GemvArgs a{};
  a.x = x;
  a.w[0] = w;
  a.w[1] = w2;
  a.out[0] = out;
  a.K = K;
  a.N = N;
  a.pos = pos;
  a.table = table;
  return launch_gemv_n<false>(epi, a, s);
}

size_t decode_attn_workspace(int L, int Hq) {
  const size_t nchunks = (size_t)(L + DA_MINCH - 1) / DA_MINCH;   // bound for every length up to L
  return nchunks * Hq * DA_PR * sizeof(float);
}

hipError_t launch_decode_attn(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, int L, int Hq, int Hkv,
                              float scale, uint16_t* o, void* ws, hipStream_t s) {
  const int ch = decode_attn_chunk(L, Hkv);
  const int nchunks = (L + ch - 1) / ch;
  float* part = reinterpret_cast<float*>(ws);
  hipLaunchKernelGGL(decode_attn_partial_kernel, dim3(nchunks, Hkv), dim3(256), 0, s, q, kc, vc, L, ch, Hq, Hkv,
                     scale * kLog2e, part);
  hipLaunchKernelGGL(decode_attn_combine_kernel, dim3(Hq), dim3(256), 0, s, part, nchunks, Hq, o);
  return hipGetLastError();
}

size_t decode_layer_workspace(int max_len, int Hq, int f) {
  const size_t vec = round_up256((size_t)Hq * DA_DH * 2);
  return 2 * vec + round_up256((size_t)f * 2) + decode_attn_workspace(max_len, Hq);
}

// One layer of a decode step, six launches: QKV (with the attention norm; K
// and V into cache row L), attention partials + combine over L + 1 rows, O
// projection added into x, gate/up (with the feed-forward norm), down added
// into x.  Workspace: q, o, h vectors, then the attention partials.
hipError_t launch_decode_layer(uint16_t* x, int d, int pos, const DecodeLayerPtrs& w, int L, int Hq, int Hkv,
                               int f, float eps, bool prenorm, const float* table, float scale, void* ws,
                               hipStream_t s) {
  const size_t vec = round_up256((size_t)Hq * DA_DH * 2);
  char* base = reinterpret_cast<char*>(ws);
  uint16_t* qv = reinterpret_cast<uint16_t*>(base);
  uint16_t* ov = reinterpret_cast<uint16_t*>(base + vec);
  uint16_t* hv = reinterpret_cast<uint16_t*>(base + 2 * vec);
  void* attn_ws = base + 2 * vec + round_up256((size_t)f * 2);
  const long kv_row = (long)Hkv * DA_DH;
  hipError_t e;
  GemvArgs a{};
  a.x = x;
  a.w[0] = w.wq;
  a.w[1] = w.wk;
  a.w[2] = w.wv;
  a.out[0] = qv;
  a.out[1] = w.k_cache + (long)L * kv_row;
  a.out[2] = w.v_cache + (long)L * kv_row;
  a.K = d;
  a.N = Hq * DA_DH;
  a.nkv = Hkv * DA_DH;
  a.pos = pos;
  a.table = table;
  a.eps = eps;
  e = prenorm ? launch_gemv_n<true>(GV_QKV, a, s) : launch_gemv_n<false>(GV_QKV, a, s);
  if (e != hipSuccess) return e;
  e = launch_decode_attn(qv, w.k_cache, w.v_cache, L + 1, Hq, Hkv, scale, ov, attn_ws, s);
  if (e != hipSuccess) return e;
  GemvArgs o{};
  o.x = ov;
  o.w[0] = w.wo;
  o.out[0] = x;
  o.K = Hq * DA_DH;
  o.N = d;
  e = launch_gemv_n<false>(GV_ADD, o, s);
  if (e != hipSuccess) return e;
  GemvArgs g{};
  g.x = x;
  g.w[0] = w.w_gate;
  g.w[1] = w.w_up;
  g.out[0] = hv;
  g.K = d;
  g.N = f;
  g.eps = eps;
  e = prenorm ? launch_gemv_n<true>(GV_SWIGLU, g, s) : launch_gemv_n<false>(GV_SWIGLU, g, s);
  if (e != hipSuccess) return e;
  GemvArgs dn{};
  dn.x = hv;
  dn.w[0] = w.w_down;
  dn.out[0] = x;
  dn.K = f;
  dn.N = d;
  return launch_gemv_n<false>(GV_ADD, dn, s);
}

}  // namespace spts
