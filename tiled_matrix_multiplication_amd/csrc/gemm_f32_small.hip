// fp32 products too small for the tiled kernels' 128x128 tiles to fill the
// chip -- the tile-count-versus-compute-unit effect of the devpress GPU
// notes, section 3.7: 256^3 is four such tiles, leaving 252 CUs idle while
// each of the four runs 128 x 128 x 256 on its own fp32 matrix unit.  Here a
// workgroup takes a 32x32 tile of C and its four waves split K in
// quarters, each running v_mfma_f32_32x32x2_f32 over its quarter straight
// from global memory (the operands of a small product stay in L2); the four
// partial tiles are summed in LDS in wave order (deterministic), then
// scaled, biased (and for the full form beta * old C and ReLU added) and
// stored.  fp32 256^3: 20.9 -> 7.4 us; 256 x 256 x 8192: 531 -> 136 us.
// (Eight or sixteen waves per tile, or the next batch's loads issued under
// the current batch's instructions, measured the same at 256^3 and slower
// for longer K: 512^3 12.0 -> 21.1 us with eight.)
//
//   C[z] = act(scale * A[z] . op(B[z]) (+ bias) (+ beta * old C[z]))
//
// Operand layout of the instruction: lane (l32, g) supplies A[m0 + l32][k]
// and B[k][n0 + l32] for k = k0 + 2c + g of instruction c -- the same k on
// both sides, so the sum is over all of K whatever the order.  Elements past
// M, N or K are read as zeros; any alignment (element loads).
#include <algorithm>

#include "tmm_internal.h"

namespace tmm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChunk = 16;   // matrix instructions per load batch

template <bool NT, bool FULL>
__global__ __launch_bounds__(256) void gemm_f32_small_kernel(GemmParams p) {
  __shared__ float red[4][32][33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t tiles_n = (p.N + 31) / 32, tiles = ((p.M + 31) / 32) * tiles_n;
  const int64_t z = blockIdx.x / tiles, t = blockIdx.x - z * tiles;
  const int64_t m0 = (t / tiles_n) * 32, n0 = (t % tiles_n) * 32;
  const float *A = (const float *)p.A + z * p.strideA;
  const float *B = (const float *)p.B + z * p.strideB;

  // this wave's quarter of K, an even length
  const int64_t kq = (((p.K + 3) / 4) + 1) & ~(int64_t)1;
  const int64_t kbeg = wave * kq, kend = std::min<int64_t>(kbeg + kq, p.K);
  const int64_t m = m0 + l32, n = n0 + l32;
  const bool mok = m < p.M, nok = n < p.N;
  const float *arow = A + (mok ? m : 0) * p.lda;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int64_t k0 = kbeg; k0 < kend; k0 += 2 * kChunk) {
    float av[kChunk], bv[kChunk];
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int64_t k = k0 + 2 * c + g;
      const bool ok = k < kend;
      av[c] = (ok && mok) ? arow[k] : 0.f;
      bv[c] = (ok && nok) ? (NT ? B[n * p.ldb + k] : B[k * p.ldb + n]) : 0.f;
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[c], bv[c], acc, 0, 0, 0);
  }

  // accumulator r of lane (l32, g): row 8 (r / 4) + 4 g + r % 4, column l32
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][8 * (r >> 2) + 4 * g + (r & 3)][l32] = acc[r];
  __syncthreads();
  float *C = (float *)p.C + z * p.strideC;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 5) + 8 * i, col = tid & 31;
    const int64_t gm = m0 + row, gn = n0 + col;
    if (gm >= p.M || gn >= p.N) continue;
    const float s = ((red[0][row][col] + red[1][row][col]) + red[2][row][col]) + red[3][row][col];
    float v = s * p.scale + (p.bias ? p.bias[gn] : 0.f);
    float *dst = C + gm * p.ldc + gn;
    if constexpr (FULL) {
      if (p.beta != 0.f) v += p.beta * *dst;
      if (p.act == 1) v = v > 0.f ? v : 0.f;
    }
    *dst = v;
  }
}

}  // namespace

hipError_t launch_gemm_f32_small(bool trans_b, const GemmParams &p, hipStream_t stream) {
  const int64_t blocks = ((p.M + 31) / 32) * ((p.N + 31) / 32) * p.batch;
  const bool full = p.beta != 0.f || p.act != 0;
  if (trans_b) {
    if (full) hipLaunchKernelGGL((gemm_f32_small_kernel<true, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((gemm_f32_small_kernel<true, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  } else {
    if (full) hipLaunchKernelGGL((gemm_f32_small_kernel<false, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((gemm_f32_small_kernel<false, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace tmm
