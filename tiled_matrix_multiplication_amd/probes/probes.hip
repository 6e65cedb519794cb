// Measurement kernels: the ceilings the library's kernels are measured
// against (declarations, contract and page citations in include/tmm_probes.h).
#include <stdint.h>

#include "tmm.h"
#include "tmm_probes.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// One wave per row: lane l loads chunks l, l + 64, ... (NL 16-byte loads,
// all issued before any is used), XOR-folded into one value.
template <int NL>
__global__ void stream_read_kernel(const char *src, int64_t rows, int64_t row_bytes, int *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const i32x4 *p = (const i32x4 *)(src + row * row_bytes) + lane;
  i32x4 v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) v[i] = __builtin_nontemporal_load(p + 64 * i);
  i32x4 x = v[0];
#pragma unroll
  for (int i = 1; i < NL; ++i) x ^= v[i];
  const int f = x[0] ^ x[1] ^ x[2] ^ x[3];
  // bf16 / fp16 / fp32 data never folds to this pattern in every lane
  if (__builtin_amdgcn_readfirstlane(f) == 0x7fc07fc1 && f == 0x7fc07fc1) *sink = f;
}

template <int SHAPE>
__global__ __launch_bounds__(512) void mfma_loop_kernel(const i32x4 *__restrict__ src, int64_t iters,
                                                         float *sink) {
  // thread gt's 24 fragments: src[24 gt .. 24 gt + 23] (the host checks the size)
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const i32x4 *q = src + gt * 24;
  i32x4 a[4][4], b[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[s][i] = q[s * 6 + i];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[s][j] = q[s * 6 + 4 + j];
  }
  float sum = 0.f;
  if constexpr (SHAPE == 0) {
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0.f};
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s][i]),
                                                                __builtin_bit_cast(bf16x8, b[s][j]), acc[i][j],
                                                                0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  } else if constexpr (SHAPE == 1) {
    // the same 128x64 block as 8x4 blocks of 16x16; per K-step s, 16
    // instructions (each row block with two of the four column blocks,
    // alternating), 64 per round: the same flops as shape 0
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * (s & 1) + jj;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a[s][i >> 1]), __builtin_bit_cast(bf16x8, b[s][jj]), acc[i][j], 0, 0, 0);
          }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sum += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  } else if constexpr (SHAPE == 2) {
    // fp8 e4m3, 32x32x64 (8 per round, 1 Mi flop): the 128x64 block as 4x2
    // accumulators, operands of 32 bytes per lane from two 16-byte fragments
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0.f};
    // 32-byte operands straight from the thread's fragments: 2 K-steps of A
    // (4 blocks) and B (2 blocks), 96 registers like the 16-bit shapes
    const i32x8 *q8 = (const i32x8 *)q;
    i32x8 a8[2][4], b8[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a8[s][i] = q8[s * 6 + i];
#pragma unroll
      for (int j = 0; j < 2; ++j) b8[s][j] = q8[s * 6 + 4 + j];
    }
    for (int64_t it = 0; it < iters; it += 4)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[s & 1][i], b8[(s >> 1) & 1][j], acc[i][j],
                                                                        0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  } else {
    // fp8 e4m3, 16x16x128 (16 per round, 1 Mi flop): 8x4 16x16 accumulators
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const i32x8 *q8 = (const i32x8 *)q;
    i32x8 a8[2][4], b8[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a8[s][i] = q8[s * 6 + i];
#pragma unroll
      for (int j = 0; j < 2; ++j) b8[s][j] = q8[s * 6 + 4 + j];
    }
    for (int64_t it = 0; it < iters; it += 4)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * (s & 1) + jj;
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8[s & 1][i >> 1], b8[(s >> 1) & 1][jj],
                                                                         acc[i][j], 0, 0, 0, 0, 0, 0);
          }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sum += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  }
  sink[gt] = sum;
}

}  // namespace

extern "C" {

int tmmp_stream_read(const void *src, int64_t rows, int64_t row_bytes, int waves_per_group, int *sink,
                     hipStream_t stream) {
  if (rows < 0 || row_bytes <= 0 || row_bytes % 1024 != 0 || row_bytes > 65536) return TMM_ERR_DIM;
  if (waves_per_group != 1 && waves_per_group != 2 && waves_per_group != 4 && waves_per_group != 8 &&
      waves_per_group != 16)
    return TMM_ERR_ARG;
  if (rows == 0) return TMM_OK;
  if (!src || !sink) return TMM_ERR_NULL;
  if ((uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0) return TMM_ERR_ALIGN;
  const int64_t groups = (rows + waves_per_group - 1) / waves_per_group;
  if (groups > 0x7fffffff) return TMM_ERR_DIM;
  const dim3 grid((unsigned)groups), block(64 * waves_per_group);
  const char *s = (const char *)src;
  switch (row_bytes / 1024) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, grid, block, 0, stream, s, rows, row_bytes, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, stream, s, rows, row_bytes, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, stream, s, rows, row_bytes, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, stream, s, rows, row_bytes, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, grid, block, 0, stream, s, rows, row_bytes, sink); break;
    case 32: hipLaunchKernelGGL(stream_read_kernel<32>, grid, block, 0, stream, s, rows, row_bytes, sink); break;
    case 64: hipLaunchKernelGGL(stream_read_kernel<64>, grid, block, 0, stream, s, rows, row_bytes, sink); break;
    default: return TMM_ERR_DIM;  // row_bytes / 1024 must be a power of two
  }
  return hipGetLastError() == hipSuccess ? TMM_OK : TMM_ERR_LAUNCH;
}

int tmmp_mfma_loop(const void *operands, int64_t operand_bytes, int shape, int64_t groups, int64_t iters,
                   float *sink, hipStream_t stream) {
  if (groups < 0 || iters < 0 || operand_bytes < (16 << 20)) return TMM_ERR_DIM;
  if (shape < 0 || shape > 3) return TMM_ERR_ARG;
  if (shape >= 2 && iters % 4 != 0) return TMM_ERR_DIM;
  if (groups == 0) return TMM_OK;
  // each of the groups x 512 threads reads its own 24 16-byte fragments
  if (groups > 0x7fffffff || operand_bytes < groups * 512 * 24 * 16) return TMM_ERR_DIM;
  if (!operands || !sink) return TMM_ERR_NULL;
  if ((uintptr_t)operands % 16 != 0 || (uintptr_t)sink % 4 != 0) return TMM_ERR_ALIGN;
  const i32x4 *src = (const i32x4 *)operands;
  const dim3 grid((unsigned)groups), block(512);
  switch (shape) {
    case 0: hipLaunchKernelGGL(mfma_loop_kernel<0>, grid, block, 0, stream, src, iters, sink); break;
    case 1: hipLaunchKernelGGL(mfma_loop_kernel<1>, grid, block, 0, stream, src, iters, sink); break;
    case 2: hipLaunchKernelGGL(mfma_loop_kernel<2>, grid, block, 0, stream, src, iters, sink); break;
    default: hipLaunchKernelGGL(mfma_loop_kernel<3>, grid, block, 0, stream, src, iters, sink); break;
  }
  return hipGetLastError() == hipSuccess ? TMM_OK : TMM_ERR_LAUNCH;
}

}  // extern "C"
