// Internal interface between the C-ABI dispatch (tmm_api.hip) and the
// kernel translation units.  Nothing here crosses the library boundary.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tmm {

// Compute units of the current device (cached per device, thread-safe).
int device_cu_count();

// GEMV launch shape pinned by the library's override (R * 100 + W), or 0.
int gemv_override();

// Convolution kernel pinned by the override: 0 none, 1 the LDS-staged
// four-wave kernel, 2 the register-direct one.
int conv_override();

// Ring depth of the four-wave kernel on 128x128 tiles pinned by the
// override: 0 none, else 4 or 8 stages.
int ring_override();

// Element formats, same numbering as tmm_dtype in include/tmm.h.
enum Fmt : int { kF32 = 0, kBF16 = 1, kF16 = 2, kF8 = 3 };

// Workgroup tile shapes of the MFMA GEMM kernel (the first kNumAutoTiles
// are chosen by shape; 256x256 runs 8 waves, the others 4; the 4-wave
// 256x256 variant is only selected by name).
enum Tile : int {
  kTile256x256 = 0,
  kTile256x128 = 1,
  kTile128x128 = 2,
  kTile256x256w4 = 3,
  kTile256x256s2 = 4,  // 256x256 on the two-stage kernel only
  kTile256x256r = 5,   // 256x256 on the ring kernel wherever it applies (also trans_b)
  kTileSkinny = 6,     // the skinny-M kernel (16-bit NT only); chosen in the dispatch
  kTile256x256q = 7,   // 256x256 on the four-wave 128x128-per-wave kernel (16-bit inputs)
  kTile256x128q = 8,   // 256x128 on the four-wave kernel (128x64 per wave)
  kTile128x128q = 9,   // 128x128 on the four-wave kernel (64x64 per wave)
  kNumAutoTiles = 3
};

struct GemmParams {
  int64_t M, N, K;
  const void *A;
  int64_t lda, strideA;
  const void *B;
  int64_t ldb, strideB;
  void *C;
  int64_t ldc, strideC;
  const float *bias;
  float scale;      // alpha: scale_a * scale_b (1 unless fp8) in the plain form
  int64_t batch;
  float beta;       // full form: + beta * old C (0: C is not read)
  int act;          // full form: 0 none, 1 ReLU, applied last
};

// Rows/columns of a workgroup tile.
inline int tile_bm(Tile t) { return (t == kTile128x128 || t == kTile128x128q) ? 128 : 256; }
inline int tile_bn(Tile t) {
  return (t == kTile256x256 || t == kTile256x256w4 || t == kTile256x256s2 || t == kTile256x256r ||
          t == kTile256x256q)
             ? 256
             : 128;
}

// Launch the tiled MFMA GEMM for one input type with the given tile shape.
// `vec` selects the 16-byte-load path (every operand row 16-byte aligned);
// otherwise element loads are used (128x128 tiles).  Returns hipSuccess or
// the launch error.
// fp32 products of few 128x128 tiles: 32x32 tiles, K split over the four
// waves of a workgroup (gemm_f32_small.hip); plain or full form.
hipError_t launch_gemm_f32_small(bool trans_b, const GemmParams &p, hipStream_t stream);

hipError_t launch_gemm_f32(Fmt c, bool trans_b, Tile tile, bool vec, const GemmParams &p,
                           hipStream_t stream);
hipError_t launch_gemm_bf16(Fmt c, bool trans_b, Tile tile, bool vec, const GemmParams &p,
                            hipStream_t stream);
hipError_t launch_gemm_f16(Fmt c, bool trans_b, Tile tile, bool vec, const GemmParams &p,
                           hipStream_t stream);
hipError_t launch_gemm_f8(Fmt c, bool trans_b, Tile tile, bool vec, const GemmParams &p,
                          hipStream_t stream);

// Skinny-M GEMM (16-bit inputs, B stored N x K, every row of A and B
// 16-byte aligned): bm x bn workgroup tiles, bm, bn in {16, 32, 64};
// vec_c allows 4-column vector stores (C aligned for them).
hipError_t launch_gemm_skinny(Fmt ab, Fmt c, int bm, int bn, bool vec_c, const GemmParams &p,
                              hipStream_t stream);

// Any-layout GEMM (16-bit inputs; A may be stored K x M): 64 x 64 tiles.
// vec_a / vec_b allow 16-byte loads (rows 16-byte aligned).
hipError_t launch_gemm_generic(Fmt ab, Fmt c, bool trans_a, bool trans_b, bool vec_a, bool vec_b,
                               const GemmParams &p, hipStream_t stream);

// 256 x 256 ring kernel with A stored K x M (16-bit inputs): every row of A
// and B 16-byte aligned, M*E and (for an N-contiguous B) N*E multiples of
// 16, K a multiple of 32.
hipError_t launch_gemm_ring_ta(Fmt ab, Fmt c, bool trans_b, const GemmParams &p, hipStream_t stream);

// Persistent short-K kernel (gemm_short_k.hip): C[z] = A[z] . B[z]^T with
// 16-bit inputs and output of the same type, K = 64 or 128, M and N
// multiples of 256, no bias, scale 1; every row and C 16-byte aligned, so
// each tile is whole and every epilogue store is a vector store.  `grid`
// workgroups (a multiple of 8) walk the tiles.
hipError_t launch_gemm_short_k(Fmt ab, const GemmParams &p, unsigned grid, hipStream_t stream);

// C = act(bias + beta * old C) (bias, beta default none) for the K == 0
// empty sum.
hipError_t launch_fill(Fmt c, const GemmParams &p, hipStream_t stream);

// C[m][n] = round(scale * (W[0][m][n] + ... + W[S-1][m][n]) + bias[n]) for
// fp32 partials W (S dense M x N planes) into C (ldc, format c) (splitk.hip).
hipError_t launch_splitk_reduce(Fmt c, int64_t M, int64_t N, int S, const float *W, void *C,
                                int64_t ldc, const float *bias, float scale, hipStream_t stream);

struct GemvParams {
  int64_t N, K;
  const void *W;
  int64_t ldw;
  const void *x;
  void *y;
  const float *bias;
};

hipError_t launch_gemv(Fmt w, Fmt y, bool vec, const GemvParams &p, hipStream_t stream);

// Y[m] = W . X[m] (+ bias) for m < M, 2 <= M <= 8: X is M x K (row pitch
// ldx), Y is M x N (row pitch ldy), W is N x K; 16-bit W and X, every row of
// W and X 16-byte aligned and K*E a multiple of 16.
struct GemvMParams {
  int64_t N, K;
  const void *W;
  int64_t ldw;
  const void *x;
  int64_t ldx;
  int64_t M;
  void *y;
  int64_t ldy;
  const float *bias;
};

hipError_t launch_gemv_multi(Fmt w, Fmt y, const GemvMParams &p, hipStream_t stream);

struct AttnParams {
  int64_t Z, Nq, Nk;
  const void *Q;
  int64_t ldq, strideQ;
  const void *K;
  int64_t ldk, strideK;
  const void *V;
  int64_t ldv, strideV;
  void *O;
  int64_t ldo, strideO;
  float scale_log2;  // scale * log2(e): scores go through exp2
};

// Fused stride-1 convolution, NHWC: out = pool(act(conv(in, w) * scale +
// bias)); in N x H x W x C, w K x R x S x C, out N x (P/pool) x (Q/pool) x K
// with P = H + 2 pad - R + 1, Q = W + 2 pad - S + 1; C % 8 == 0.
struct ConvParams {
  int64_t N;
  int H, W, C, K, R, S, pad, pool, relu;
  const void *in;
  const void *w;
  const float *scale;
  const float *bias;
  void *out;
};

hipError_t launch_conv(Fmt in, Fmt out, const ConvParams &p, hipStream_t stream);

// Fused attention forward (attention.hip); D is 64 or 128, in is kF16 or
// kBF16, out is in or kF32 (the host has checked all of it).
hipError_t launch_attention(Fmt in, Fmt out, int D, const AttnParams &p, hipStream_t stream);

}  // namespace tmm
