// GEMM for any operand layout, C = act(alpha * op(A) . op(B) + bias + beta
// * old C), with op = identity or transpose per operand: the BLAS interface
// of the "GEMM to FlashAttention" page (transa / transb, alpha, beta, lda /
// ldb / ldc) with the ReLU unit of the Lecture 27 notes (section 2.1).  The
// main kernels take A with K contiguous (rows of A); this one also takes A
// stored K x M (a transposed operand, as in the weight gradient X^T . dY),
// for bf16 / fp16 inputs.
//
// Layout of the work: 64 x 64 output tiles, 4 waves as 2 x 2, each 32 x 32 =
// 2 x 2 v_mfma_f32_16x16x32 blocks; K steps of 32.  Each step moves the A
// and B tiles into LDS as K-contiguous rows (A: 64 rows of op(A), B: 64 rows
// of op(B)^T, 80-byte pitch): a K-contiguous operand with one 16-byte load
// and one 16-byte LDS write per thread, an M- (N-) contiguous one with one
// 16-byte load of 8 neighbouring rows of op and eight 2-byte LDS writes that
// transpose it.  Fragments come back with 16-byte LDS reads (lane l: row
// l % 16 of its block, K elements 8 (l / 16) .. +7).  Elements past M, N or
// K are read as zero; outputs past M or N are not stored.
#include <stdint.h>

#include "load_words.h"
#include "tmm_internal.h"

namespace tmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBT = 64;     // tile rows and columns
constexpr int kBK = 32;     // K per step
constexpr int kPitch = 40;  // LDS row pitch in elements (80 bytes)

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

template <int F>
__device__ __forceinline__ float value16(uint16_t u) {
  if constexpr (F == kBF16) return __uint_as_float((uint32_t)u << 16);
  else return (float)__builtin_bit_cast(_Float16, u);
}

template <int F>
__device__ __forceinline__ uint16_t round16(float v) {
  if constexpr (F == kBF16)
    return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v, 0.f}, bf16x2)) & 0xffffu);
  else
    return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v, 0.f}, f16x2)) & 0xffffu);
}

// load8_u16_words: the misaligned 16-bit piece loader of load_words.h.

// 8 consecutive elements X[r][c .. c+7] of a row-major (rows x cols, ld)
// matrix, zero outside it; one 16-byte load when whole and `vec`, else
// word loads of the valid part.
__device__ __forceinline__ i32x4 load8(const uint16_t *X, int64_t ld, int64_t rows, int64_t cols,
                                       int64_t r, int64_t c, bool vec) {
  if (r < rows && c + 8 <= cols && vec) return *(const i32x4 *)(X + r * ld + c);
  const int64_t left = r < rows ? cols - c : 0;
  const int nv = left <= 0 ? 0 : (left >= 8 ? 8 : (int)left);
  return load8_u16_words((const char *)(X + r * ld + c), nv);
}

// One operand tile into LDS as 64 K-contiguous rows of kPitch elements.
// KC: the operand is stored with K contiguous (rows = tile rows, e.g. A, or
// B stored N x K); otherwise it is stored K x rows and is transposed here.
template <bool KC>
__device__ __forceinline__ void stage(uint16_t *T, const uint16_t *X, int64_t ld, int64_t nrows,
                                      int64_t K, int64_t r0, int64_t k0, bool vec, int tid) {
  if constexpr (KC) {
    const int row = tid >> 2, kc = (tid & 3) * 8;
    const i32x4 v = load8(X, ld, nrows, K, r0 + row, k0 + kc, vec);
    *(i32x4 *)(T + row * kPitch + kc) = v;
  } else {
    const int kr = tid >> 3, rc = (tid & 7) * 8;
    const i32x4 v = load8(X, ld, K, nrows, k0 + kr, r0 + rc, vec);
#pragma unroll
    for (int e = 0; e < 8; ++e) T[(rc + e) * kPitch + kr] = (uint16_t)((uint32_t)v[e >> 1] >> (16 * (e & 1)));
  }
}

template <int AB, int CT, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GemmParams p, int vec_a, int vec_b) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBT * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBT * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, kq = lane >> 4;

  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t tiles_m = (M + kBT - 1) / kBT, tiles_n = (N + kBT - 1) / kBT;
  const int64_t tiles = tiles_m * tiles_n;
  const int64_t bid = remap_xcd(blockIdx.x, (int64_t)gridDim.x);
  const int64_t z = bid / tiles;
  const int64_t t = bid - z * tiles;
  const int64_t tm = t % tiles_m, tn = t / tiles_m;
  const int64_t m0 = tm * kBT, n0 = tn * kBT;
  const uint16_t *A = (const uint16_t *)p.A + z * p.strideA;
  const uint16_t *B = (const uint16_t *)p.B + z * p.strideB;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    stage<!TA>(As, A, p.lda, M, K, m0, k0, vec_a != 0, tid);
    stage<TB>(Bs, B, p.ldb, N, K, n0, k0, vec_b != 0, tid);
    __syncthreads();
    i32x4 fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      fa[i] = *(const i32x4 *)(As + (wm * 32 + 16 * i + r16) * kPitch + 8 * kq);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[j] = *(const i32x4 *)(Bs + (wn * 32 + 16 * j + r16) * kPitch + 8 * kq);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mma<AB>(fa[i], fb[j], acc[i][j]);
    __syncthreads();
  }

  // register r of block (i, j): row 16 i + 4 kq + r, column 16 j + r16
  char *C = (char *)p.C + z * p.strideC * (CT == kF32 ? 4 : 2);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t col = n0 + wn * 32 + 16 * j + r16;
    if (col >= N) continue;
    const float bv = p.bias ? p.bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * 32 + 16 * i + 4 * kq + r;
        if (row >= M) continue;
        const int64_t idx = row * p.ldc + col;
        float v = acc[i][j][r] * p.scale + bv;
        if constexpr (CT == kF32) {
          if (p.beta != 0.f) v += p.beta * ((const float *)C)[idx];
          if (p.act == 1) v = v > 0.f ? v : 0.f;
          ((float *)C)[idx] = v;
        } else {
          if (p.beta != 0.f) v += p.beta * value16<CT>(((const uint16_t *)C)[idx]);
          if (p.act == 1) v = v > 0.f ? v : 0.f;
          ((uint16_t *)C)[idx] = round16<CT>(v);
        }
      }
  }
}

template <int AB, int CT, bool TA, bool TB>
hipError_t launch_one(const GemmParams &p, bool vec_a, bool vec_b, hipStream_t stream) {
  const int64_t tiles = ((p.M + kBT - 1) / kBT) * ((p.N + kBT - 1) / kBT) * p.batch;
  hipLaunchKernelGGL((gemm_generic_kernel<AB, CT, TA, TB>), dim3((unsigned)tiles), dim3(256), 0, stream, p,
                     vec_a ? 1 : 0, vec_b ? 1 : 0);
  return hipGetLastError();
}

template <int AB, int CT>
hipError_t launch_layouts(bool ta, bool tb, const GemmParams &p, bool va, bool vb, hipStream_t s) {
  if (ta) return tb ? launch_one<AB, CT, true, true>(p, va, vb, s) : launch_one<AB, CT, true, false>(p, va, vb, s);
  return tb ? launch_one<AB, CT, false, true>(p, va, vb, s) : launch_one<AB, CT, false, false>(p, va, vb, s);
}

}  // namespace

hipError_t launch_gemm_generic(Fmt ab, Fmt c, bool trans_a, bool trans_b, bool vec_a, bool vec_b,
                               const GemmParams &p, hipStream_t stream) {
  if (ab == kBF16) return c == kF32 ? launch_layouts<kBF16, kF32>(trans_a, trans_b, p, vec_a, vec_b, stream)
                                    : launch_layouts<kBF16, kBF16>(trans_a, trans_b, p, vec_a, vec_b, stream);
  if (ab == kF16) return c == kF32 ? launch_layouts<kF16, kF32>(trans_a, trans_b, p, vec_a, vec_b, stream)
                                   : launch_layouts<kF16, kF16>(trans_a, trans_b, p, vec_a, vec_b, stream);
  return hipErrorInvalidValue;
}

}  // namespace tmm
