// Skinny GEMM on gfx950 matrix cores: C = scale * A . B^T (+ bias) with B
// stored N x K (a linear layer's weight, output features x input
// features) and few rows M, the batched-decode end of the batch-size table
// on the "GEMM to FlashAttention" page (a 4096 x 4096 weight at batch 1 ...
// 4096: memory-bound up to a few hundred rows, then the transition to
// compute-bound).  At these shapes the 256x256 / 128x128 tiles of the main
// kernels give a handful of workgroups and leave most CUs idle while the
// whole weight still has to stream from HBM once.
//
// Layout of the work:
//   * workgroup tiles of BM x BN outputs with BM, BN in {16, 32, 64}, picked
//     by the host so that there are at least as many tiles as CUs; tile
//     (tm, tn) is visited with tm fastest and workgroups are mapped to XCDs
//     in contiguous runs, so the row panels that share a weight panel run
//     together on one XCD and the weight comes from HBM once;
//   * the NW waves of a workgroup (16 for the small tiles, 8 for the wide
//     ones) split K: wave w takes the 64-element K steps w, w + NW, ...
//     (together they read contiguous row pieces), so the weight panel
//     streams through all of them at once with 48-128 KiB of loads in
//     flight per CU.  A step is two 32-element pieces, one matrix
//     instruction each, loaded back to back, so the 64-byte pieces of a row
//     that one wave requests make whole 128-byte lines (one piece per step
//     measured 9-12 % slower at M = 4 ... 256);
//   * both operands are K-contiguous rows, which is what the MFMA operands
//     want: 16-byte global loads go straight into registers (no LDS, no
//     transposes), P steps ahead of their use;
//   * v_mfma_f32_16x16x32 (bf16/f16): lane l supplies row l % 16 and K
//     elements 8 (l / 16) .. +7 of both operands and receives rows
//     4 (l / 16) .. +3 of column l % 16;
//   * the NW partial tiles are summed by a fixed tree through LDS (waves
//     w and w + h for h = NW/2, NW/4, ..., 1; the result does not depend
//     on timing), then scale, bias, one nearest-even rounding and row-wise
//     stores (in the full form also + beta * old C and ReLU before the
//     rounding).
// Rows past M (columns past N) read the last valid row and are not stored;
// a K tail (K % 64) is read element by element with zero fill, one 32-wide
// piece at a time.
#include <stdint.h>

#include "tmm_internal.h"

namespace tmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kKS = 32;   // K elements per matrix instruction

__device__ __forceinline__ int64_t remap_xcd(int64_t pid, int64_t n) {
  const int64_t per = n >> 3;
  if (pid >= (per << 3)) return pid;
  return (pid & 7) * per + (pid >> 3);
}

template <int AB>
__device__ __forceinline__ f32x4 mma(i32x4 a, i32x4 b, f32x4 c) {
  if constexpr (AB == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats as two 16-bit values of format F, nearest-even.
template <int F>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (F == kBF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
template <int F>
__device__ __forceinline__ uint16_t to16(float v) {
  return (uint16_t)(pack2<F>(v, 0.f) & 0xffffu);
}

// 8 consecutive 16-bit elements of a row from element k on, zero at and past
// K (the K tail).
__device__ __forceinline__ i32x4 load_tail(const uint16_t *row, int64_t k, int64_t K) {
  uint16_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = (k + j < K) ? row[k + j] : (uint16_t)0;
  i32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = (int)((uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16));
  return v;
}

template <int AB, int CT, int BM, int BN, int P, int NW, int KP>
__global__ __launch_bounds__(64 * NW, 1) void gemm_skinny_kernel(GemmParams p, int64_t tiles_m,
                                                                  int64_t tiles_n, int vec_c) {
  constexpr int kWaves = NW;
  constexpr int FM = BM / 16, FN = BN / 16;
  // floats per LDS row: a store or tree-step read of one accumulator
  // register touches 16 consecutive floats of 4 rows 4 apart; with the pitch
  // 4 more than a multiple of 16 those rows start 16 banks apart, so the
  // four 16-lane groups cover all 64 banks (the earlier BN + 16 put all four
  // on the same 16 banks: 50 % of LDS-active cycles were bank conflicts at
  // M = 256)
  constexpr int PITCH = BN + 4;
  constexpr int CE = CT == kF32 ? 4 : 2;
  __shared__ __attribute__((aligned(16))) float red[NW / 2][BM][PITCH];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kq = lane >> 4;

  const int64_t tiles = tiles_m * tiles_n;
  const int64_t bid = remap_xcd(blockIdx.x, (int64_t)gridDim.x);
  const int64_t z = bid / tiles;
  const int64_t t = bid - z * tiles;
  const int64_t tn = t / tiles_m, tm = t - tn * tiles_m;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t M = p.M, N = p.N, K = p.K;

  const uint16_t *Az = (const uint16_t *)p.A + z * p.strideA;
  const uint16_t *Bz = (const uint16_t *)p.B + z * p.strideB;
  const uint16_t *arow[FM];
  const uint16_t *brow[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int64_t r = m0 + 16 * f + r16;
    arow[f] = Az + (r < M ? r : M - 1) * p.lda;
  }
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int64_t r = n0 + 16 * f + r16;
    brow[f] = Bz + (r < N ? r : N - 1) * p.ldb;
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Full K steps of this wave: s = wave + NW i, i < cnt.  Ring of P steps of
  // fragments; step i sits in slot i % P.
  // A wave's step is KP consecutive 32-element pieces: with KP = 2 the two
  // 64-byte pieces of each row it loads make one whole 128-byte line.
  constexpr int KSTEP = kKS * KP;
  const int64_t nfull = K / KSTEP;
  const int64_t cnt = nfull > wave ? (nfull - wave + kWaves - 1) / kWaves : 0;
  i32x4 fa[P][KP][FM], fb[P][KP][FN];
  auto load = [&](int64_t i, int slot) __attribute__((always_inline)) {
    const int64_t k = (wave + kWaves * i) * KSTEP + 8 * kq;
#pragma unroll
    for (int h = 0; h < KP; ++h) {
#pragma unroll
      for (int f = 0; f < FM; ++f) fa[slot][h][f] = *(const i32x4 *)(arow[f] + k + h * kKS);
#pragma unroll
      for (int f = 0; f < FN; ++f) fb[slot][h][f] = *(const i32x4 *)(brow[f] + k + h * kKS);
    }
  };
  auto compute1 = [&](const i32x4 (&a)[FM], const i32x4 (&b)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mma<AB>(a[i], b[j], acc[i][j]);
  };
  auto compute = [&](const i32x4 (&a)[KP][FM], const i32x4 (&b)[KP][FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < KP; ++h) compute1(a[h], b[h]);
  };

#pragma unroll
  for (int q = 0; q < P; ++q)
    if (q < cnt) load(q, q);
  int64_t i = 0;
  for (; i + P <= cnt; i += P) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      compute(fa[q], fb[q]);
      if (i + q + P < cnt) load(i + q + P, q);
    }
  }
#pragma unroll
  for (int q = 0; q < P; ++q)
    if (i + q < cnt) compute(fa[q], fb[q]);

  // K tail past the whole steps: up to KP partial pieces, owned by the wave
  // whose turn it is.
  if (K % KSTEP != 0 && wave == (int)(nfull % kWaves)) {
    for (int64_t k0 = nfull * KSTEP; k0 < K; k0 += kKS) {
      const int64_t k = k0 + 8 * kq;
      i32x4 a[FM], b[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f) a[f] = load_tail(arow[f], k, K);
#pragma unroll
      for (int f = 0; f < FN; ++f) b[f] = load_tail(brow[f], k, K);
      compute1(a, b);
    }
  }

  // Tree sum of the partial tiles: at half-width h, waves h .. 2h-1 store
  // theirs (register r of (i, j) is row 16 i + 4 kq + r, column 16 j + r16)
  // and waves 0 .. h-1 add their partner's; wave 0 ends with the total and
  // stores it to buffer 0.
#pragma unroll
  for (int h = NW / 2; h >= 1; h >>= 1) {
    if (wave >= h && wave < 2 * h) {
#pragma unroll
      for (int fi = 0; fi < FM; ++fi)
#pragma unroll
        for (int fj = 0; fj < FN; ++fj)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[wave - h][16 * fi + 4 * kq + r][16 * fj + r16] = acc[fi][fj][r];
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int fi = 0; fi < FM; ++fi)
#pragma unroll
        for (int fj = 0; fj < FN; ++fj)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[fi][fj][r] += red[wave][16 * fi + 4 * kq + r][16 * fj + r16];
    }
    __syncthreads();
  }
  if (wave == 0) {
#pragma unroll
    for (int fi = 0; fi < FM; ++fi)
#pragma unroll
      for (int fj = 0; fj < FN; ++fj)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[0][16 * fi + 4 * kq + r][16 * fj + r16] = acc[fi][fj][r];
  }
  __syncthreads();

  // Scale, bias, round, store four consecutive columns per thread.
  char *Cz = (char *)p.C + z * p.strideC * CE;
  constexpr int G4 = BN / 4;             // column quads per row
  constexpr int QUADS = BM * G4;
#pragma unroll
  for (int g0 = 0; g0 < QUADS; g0 += 64 * NW) {
    const int g = g0 + (int)threadIdx.x;
    if (QUADS % (64 * NW) != 0 && g >= QUADS) break;
    const int row = g / G4, c4 = (g - row * G4) * 4;
    const int64_t gr = m0 + row, gc = n0 + c4;
    if (gr >= M || gc >= N) continue;
    const f32x4 v = *(const f32x4 *)&red[0][row][c4];
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = v[j] * p.scale;
      if (p.bias && gc + j < N) o[j] += p.bias[gc + j];
    }
    char *dst = Cz + (gr * p.ldc + gc) * CE;
    if (p.beta != 0.f) {   // full form: + beta * old C
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (gc + j >= N) break;
        if constexpr (CT == kF32)
          o[j] += p.beta * ((const float *)dst)[j];
        else if constexpr (CT == kBF16)
          o[j] += p.beta * __uint_as_float((uint32_t)((const uint16_t *)dst)[j] << 16);
        else
          o[j] += p.beta * (float)__builtin_bit_cast(_Float16, ((const uint16_t *)dst)[j]);
      }
    }
    if (p.act == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = o[j] > 0.f ? o[j] : 0.f;
    }
    if (vec_c && gc + 4 <= N) {
      if constexpr (CT == kF32)
        *(f32x4 *)dst = f32x4{o[0], o[1], o[2], o[3]};
      else
        *(i32x2 *)dst = i32x2{(int)pack2<CT>(o[0], o[1]), (int)pack2<CT>(o[2], o[3])};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (gc + j >= N) break;
        if constexpr (CT == kF32)
          ((float *)dst)[j] = o[j];
        else
          ((uint16_t *)dst)[j] = to16<CT>(o[j]);
      }
    }
  }
}

template <int AB, int CT, int BM, int BN, int P, int NW, int KP = 2>
hipError_t launch_one(const GemmParams &p, int vec_c, hipStream_t stream) {
  const int64_t tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int64_t blocks = tiles_m * tiles_n * p.batch;
  hipLaunchKernelGGL((gemm_skinny_kernel<AB, CT, BM, BN, P, NW, KP>), dim3((unsigned)blocks), dim3(64 * NW),
                     0, stream, p, tiles_m, tiles_n, vec_c);
  return hipGetLastError();
}

// Prefetch depth P (in two-piece steps) and waves NW per tile: registers
// within the 128 (NW = 16) or 256 (NW = 8) a wave may hold without
// spilling, 48-128 KiB of B loads in flight per workgroup.
template <int AB, int CT>
hipError_t launch_typed(int bm, int bn, const GemmParams &p, int vec_c, hipStream_t s) {
  if (bm == 16) {
    if (bn == 16) return launch_one<AB, CT, 16, 16, 6, 16>(p, vec_c, s);
    if (bn == 32) return launch_one<AB, CT, 16, 32, 3, 16>(p, vec_c, s);
    return launch_one<AB, CT, 16, 64, 1, 16>(p, vec_c, s);
  }
  if (bm == 32) {
    if (bn == 16) return launch_one<AB, CT, 32, 16, 3, 16>(p, vec_c, s);
    if (bn == 32) return launch_one<AB, CT, 32, 32, 2, 16>(p, vec_c, s);
    return launch_one<AB, CT, 32, 64, 2, 8>(p, vec_c, s);
  }
  if (bn == 16) return launch_one<AB, CT, 64, 16, 1, 16>(p, vec_c, s);
  if (bn == 32) return launch_one<AB, CT, 64, 32, 2, 8>(p, vec_c, s);
  return launch_one<AB, CT, 64, 64, 1, 8>(p, vec_c, s);
}

}  // namespace

hipError_t launch_gemm_skinny(Fmt ab, Fmt c, int bm, int bn, bool vec_c, const GemmParams &p,
                              hipStream_t stream) {
  const int v = vec_c ? 1 : 0;
  if (ab == kBF16) return c == kF32 ? launch_typed<kBF16, kF32>(bm, bn, p, v, stream)
                                    : launch_typed<kBF16, kBF16>(bm, bn, p, v, stream);
  if (ab == kF16) return c == kF32 ? launch_typed<kF16, kF32>(bm, bn, p, v, stream)
                                   : launch_typed<kF16, kF16>(bm, bn, p, v, stream);
  return hipErrorInvalidValue;
}

}  // namespace tmm
