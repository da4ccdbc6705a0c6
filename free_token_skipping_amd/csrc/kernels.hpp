// Internal launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Every launcher enqueues on the given stream and returns the
// launch status; shapes have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spts {

// ------------------------------------------------------------------ GEMM
// C = A * B^T, A [m, k] bf16 (rows optionally gathered), B [n, k] bf16.
enum GemmEpilogue : int {
  EPI_STORE = 0,   // bf16 out[o(i), c] (= or +=), o(i) = out_rows ? out_rows[i] : i
  EPI_ROPE = 1,    // bf16 out with rotary embedding on 128-wide heads
  EPI_SWIGLU = 2,  // bf16 out = silu(A Wg^T) * (A Wu^T); b0 = Wg, b1 = Wu
  EPI_SPLIT = 3,   // fp32 result t written as bf16 pair hi=bf16(t), lo=bf16(t-hi)
  EPI_SUMSQ = 4,   // fp32 out[i, tile_n] = sum over the tile's 256 columns of c^2
  EPI_PARTIAL = 5, // split-K pass: fp32 partial[ks][i][c] (internal)
  EPI_KV = 6,      // two-part B: columns < n0 from b0 into out (RoPE if rope_table),
                   // the rest from b1 into out2 (ldc2 columns), both bf16
  EPI_SWIGLU_SPLIT = 7,  // as SWIGLU, the fp32 result h written as bf16 pair: hi = bf16(h)
                         // at column c, lo = bf16(h - hi) at column f + c (f = n / 2)
  EPI_QUAD = 8,    // fp32 out[(i * tiles_n + tile_n) * ksplit + kslice] = sum over the tile's
                   // columns c of C[i, c] * t[i, c] for this k-slice's part of C, t read from
                   // tperm in the lane order of quad_perm (no gather, no tail split)
};

struct GemmArgs {
  const uint16_t* a;        // A base
  const int32_t* a_rows;    // gather rows of A (nullable)
  int m, k, lda;
  const uint16_t* b0;       // B (or gate weight)
  const uint16_t* b1;       // up weight (SWIGLU only)
  int ldb;
  int kwrap;                // if > 0: B column = (k index) mod kwrap
  int n;                    // B rows covered (SWIGLU: output columns * 2)
  void* out;
  int ldc;
  const int32_t* out_rows;  // scatter rows of out (nullable)
  int accumulate;
  const int32_t* pos;       // ROPE: original position per A row (indexed like A rows)
  const float* rope_table;  // ROPE: [max_pos, 64, 2]
  int n0;                   // KV: columns taken from b0 (a multiple of 256)
  void* out2;               // KV: output of the b1 columns
  int ldc2;
  float* partial;           // split-K / tail-piece workspace (nullable: never split)
  size_t partial_bytes;
  int ksplit;               // set by the launcher
  // Tail split, set by the launcher (tail_tiles == 0: off).  Logical tiles
  // below tail_full run whole; each of the last tail_tiles tiles is cut along
  // k into tail_np pieces whose fp32 sums a second launch adds and finishes.
  // tail_ends == 0: tail_np equal pieces, one workgroup each.  tail_ends > 0:
  // a head [0, tail_kx) per workgroup, and each remaining workgroup takes the
  // ends [tail_kx, KT) of up to tail_ends tiles.
  int tail_full, tail_tiles, tail_np, tail_ends, tail_kx;
  int split3;               // EPI_SPLIT: also write the hi half again at column 2n + c
  float* tperm;             // EPI_SPLIT: if set, also the fp32 result in quad_perm order;
                            // EPI_QUAD: the row factors t, in that order
};

// Offset (floats) of element (row, col) of an [m, n] fp32 matrix stored in the
// register order of a 256 x 256 GEMM tile: tile (row / 256, col / 256), then
// wave row block, 16-row group, wave column block, 16-column group, lane
// (16 * column quad + row within the group), element.  One 16-byte load per
// lane and accumulator tile reads a contiguous KiB per wave.  Rows are padded
// to a multiple of 256: the buffer holds ceil(m / 256) * 256 * n floats.
__host__ __device__ inline long quad_perm(int row, int col, int n) {
  const int tm = row >> 8, rr = row & 255, tn = col >> 8, cc = col & 255;
  const long blk = ((((long)tm * (n >> 8) + tn) * 4 + (rr >> 6)) * 4 + ((rr >> 4) & 3)) * 2 + (cc >> 7);
  return ((blk * 8 + ((cc >> 4) & 7)) * 64 + (((cc >> 2) & 3) * 16 + (rr & 15))) * 4 + (cc & 3);
}

// Split count the launcher would use for this problem (1 = no split) and the
// workspace it then needs (split-K slices or tail pieces, whichever the
// launcher picks; 0 when it runs the problem unsplit).
int gemm_ksplit(int m, int k, int n, int epilogue);
size_t gemm_split_workspace(int m, int k, int n, int epilogue);
// k-slices of an EPI_QUAD launch: each writes its own partial row sums
int gemm_quad_ksplit(int m, int k, int n);
hipError_t launch_gemm(const GemmArgs& g, int epilogue, hipStream_t s);

// ------------------------------------------------------------ attention
hipError_t launch_probe_bf16(const uint16_t* q, const uint16_t* k, int n, int P, int Hq, int Hkv,
                             float scale, float* scores, void* ws, hipStream_t s);
hipError_t launch_probe_f32(const float* q, const float* k, int n, int P, int Hq, int Hkv, int dh,
                            float scale, float* scores, void* ws, hipStream_t s);
size_t probe_workspace(int n, int P, int Hq);

hipError_t launch_attn_bf16(const uint16_t* q, const int32_t* idx, const uint16_t* k,
                            const uint16_t* v, int kq, int n, int Hq, int Hkv, float scale,
                            uint16_t* o, hipStream_t s);
hipError_t launch_attn_f32(const float* q, const int32_t* idx, const float* k, const float* v,
                           int kq, int n, int Hq, int Hkv, int dh, float scale, float* o,
                           hipStream_t s);

// --------------------------------------------------------------- select
size_t topk_workspace(int n);
// most scores one selection takes (row indices and grid strides stay in 32 bits)
constexpr int kTopkMaxN = 1 << 30;
// s_b == nullptr: rank s_a; else fuse s_a and s_b by MaxNorm-Add (multiply == false)
// or by their product (multiply == true)
hipError_t launch_topk(const float* s_a, const float* s_b, float w_a, float w_b, bool multiply, int n,
                       int k, int n_forced, int32_t* idx, float* fused_out, void* ws, hipStream_t s);
// launch_topk with the key storage in a static per-GPU device array instead
// of a workspace: no allocation; n <= kTopkNoallocMaxN (else hipErrorInvalidValue)
constexpr int kTopkNoallocMaxN = 1 << 20;
hipError_t launch_topk_noalloc(const float* s_a, const float* s_b, float w_a, float w_b, bool multiply, int n,
                               int k, int n_forced, int32_t* idx, float* fused_out, hipStream_t s);
// one workgroup per score row (rows of at most 1024 * 32 scores, keys in registers)
hipError_t launch_topk_batched(const float* s, long s_stride, int batch, int n, int k, int n_forced, int32_t* idx,
                               long idx_stride, hipStream_t st);

// -------------------------------------------------------------- decode
// y = x W^T for one row x [K]; epi 0 store, 1 RoPE at pos (pairs c, c+64 of
// 128-wide heads), 2 SwiGLU (w = gate, w2 = up), 3 residual add into out.
bool gemv_supported_k(int K);
hipError_t launch_gemv(const uint16_t* x, const uint16_t* w, const uint16_t* w2, int K, int N, uint16_t* out,
                       int epi, int pos, const float* table, hipStream_t s);
size_t decode_attn_workspace(int L, int Hq);
hipError_t launch_decode_attn(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, int L, int Hq, int Hkv,
                              float scale, uint16_t* o, void* ws, hipStream_t s);
// one layer of a decode step (projections, attention over cache rows 0..L
// after writing row L, feed-forward); weights as in spts_decode_step
struct DecodeLayerPtrs {
  const uint16_t *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
  uint16_t *k_cache, *v_cache;
};
size_t decode_layer_workspace(int max_len, int Hq, int f);
hipError_t launch_decode_layer(uint16_t* x, int d, int pos, const DecodeLayerPtrs& w, int L, int Hq, int Hkv,
                               int f, float eps, bool prenorm, const float* table, float scale, void* ws,
                               hipStream_t s);

// ------------------------------------------------------------- row ops
hipError_t launch_gather(const void* src, const int32_t* idx, int k, long row_bytes, void* dst,
                         hipStream_t s);
hipError_t launch_scatter(const void* src, const int32_t* idx, int k, long row_bytes, void* dst,
                          hipStream_t s);
hipError_t launch_scatter_add_bf16(const uint16_t* src, const int32_t* idx, int k, int row_elems,
                                   uint16_t* dst, hipStream_t s);
hipError_t launch_scatter_add_f32(const float* src, const int32_t* idx, int k, int row_elems,
                                  float* dst, hipStream_t s);
hipError_t launch_scatter_add_i32(const int32_t* src, const int32_t* idx, int k, int row_elems,
                                  int32_t* dst, hipStream_t s);
hipError_t launch_rmsnorm(const uint16_t* x, int n, int d, float eps, uint16_t* out, hipStream_t s);
hipError_t launch_rope_table(int max_pos, int dh, double theta, float* table, hipStream_t s);
hipError_t launch_rowsum_sqrt(const float* partial, int n, int parts, float* out, hipStream_t s);
// Gram operand of the LTP proxy's second factor: G = V V^T (r x r) from
// v_t = V^T [d, r] bf16, accumulated in fp64, written as bf16 rows
// [hi(G) | hi(G) | lo(G)] of width 3r (gcat [r, 3r])
hipError_t launch_ltp_gram(const uint16_t* v_t, int d, int r, uint16_t* gcat, hipStream_t s);

}  // namespace spts
