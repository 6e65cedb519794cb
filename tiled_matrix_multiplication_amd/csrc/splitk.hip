// Second pass of the split-K product (tmm_gemm_splitk): the S fp32 partial
// products W[s] (dense M x N planes, s = K slice) are summed in the fixed
// order W[0] + W[1] + ... + W[S-1], then scaled, the bias added and the
// result rounded once to the output format (nearest-even), as the one-pass
// epilogue does: C = scale * sum + bias, the linear-layer formula of the
// "GEMM to FlashAttention" page.
//
// HBM-bound: S*M*N*4 bytes read (the partials, streamed with non-temporal
// loads: each is read once) and M*N output elements written.  A thread
// takes 4 consecutive columns of a row: one 16-byte load per plane when the
// rows are 16-byte aligned (N % 4 == 0), a 4- or 8-byte store when C and its
// pitch allow; otherwise element by element with the same order of sums.
#include <stdint.h>

#include <algorithm>

#include "gemm_mfma.h"
#include "tmm_internal.h"

namespace tmm {
namespace {

using gemm_detail::f32x4;
using gemm_detail::out_bits;

template <int CT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *W, int64_t M, int64_t N, int S,
                                                            char *C, int64_t ldc, const float *bias,
                                                            float scale, int vec_w, int vec_c) {
  constexpr int CE = CT == kF32 ? 4 : 2;
  const int64_t qpr = (N + 3) >> 2;     // 4-column quads per row
  const int64_t total = M * qpr;
  const int64_t plane = M * N;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const int64_t m = q / qpr, n0 = (q - m * qpr) * 4;
    const float *w = W + m * N + n0;
    const bool whole = n0 + 4 <= N;
    float v[4];
    if (vec_w && whole) {
      f32x4 a = __builtin_nontemporal_load((const f32x4 *)w);
      for (int s = 1; s < S; ++s) {
        const f32x4 b = __builtin_nontemporal_load((const f32x4 *)(w + s * plane));
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = a[e] + b[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = a[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = 0.f;
        if (n0 + e < N) {
          a = w[e];
          for (int s = 1; s < S; ++s) a = a + w[s * plane + e];
        }
        v[e] = a;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = v[e] * scale + ((bias && n0 + e < N) ? bias[n0 + e] : 0.f);
    char *dst = C + (m * ldc + n0) * CE;
    if (vec_c && whole) {
      if constexpr (CT == kF32) {
        *(f32x4 *)dst = f32x4{v[0], v[1], v[2], v[3]};
      } else {
        const uint64_t b = (uint64_t)out_bits<CT>(v[0]) | ((uint64_t)out_bits<CT>(v[1]) << 16) |
                           ((uint64_t)out_bits<CT>(v[2]) << 32) | ((uint64_t)out_bits<CT>(v[3]) << 48);
        *(uint64_t *)dst = b;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n0 + e >= N) break;
        if constexpr (CT == kF32) ((float *)dst)[e] = v[e];
        else ((uint16_t *)dst)[e] = (uint16_t)out_bits<CT>(v[e]);
      }
    }
  }
}

template <int CT>
hipError_t launch_typed(int64_t M, int64_t N, int S, const float *W, void *C, int64_t ldc,
                        const float *bias, float scale, hipStream_t stream) {
  constexpr int CE = CT == kF32 ? 4 : 2;
  const int64_t quads = M * ((N + 3) / 4);
  const int64_t cap = (int64_t)device_cu_count() * 16;   // grid-stride beyond 16 workgroups per CU
  const int64_t blocks = std::min<int64_t>((quads + 255) / 256, cap);
  const int vec_w = N % 4 == 0 ? 1 : 0;
  const int vec_c = ((uintptr_t)C % (4 * CE)) == 0 && ldc % 4 == 0 ? 1 : 0;
  hipLaunchKernelGGL((splitk_reduce_kernel<CT>), dim3((unsigned)blocks), dim3(256), 0, stream, W, M, N, S,
                     (char *)C, ldc, bias, scale, vec_w, vec_c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_splitk_reduce(Fmt c, int64_t M, int64_t N, int S, const float *W, void *C, int64_t ldc,
                                const float *bias, float scale, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (c == kF32) return launch_typed<kF32>(M, N, S, W, C, ldc, bias, scale, stream);
  if (c == kBF16) return launch_typed<kBF16>(M, N, S, W, C, ldc, bias, scale, stream);
  if (c == kF16) return launch_typed<kF16>(M, N, S, W, C, ldc, bias, scale, stream);
  return hipErrorInvalidValue;
}

}  // namespace tmm
