// Second pass of the split-K product (tmm_gemm_splitk): the S fp32 partial
// products W[s] (dense M x N planes, s = K slice) are summed in the fixed
// order W[0] + W[1] + ... + W[S-1], then scaled, the bias added and the
// result rounded once to the output format (nearest-even), as the one-pass
// epilogue does: C = scale * sum + bias, the linear-layer formula of the
// "GEMM to FlashAttention" page.
//
// HBM-bound: S*M*N*4 bytes read (the partials, each read once) and M*N
// output elements written.  A thread takes 4 consecutive columns of a row:
// one 16-byte load per plane when the rows are 16-byte aligned (N % 4 == 0),
// a 4- or 8-byte store when C and its pitch allow; otherwise element by
// element with the same order of sums.  The planes' loads are all issued
// before the first add (S a compile-time constant up to 8, else groups of
// 8), where a loop loading one plane and waiting before the next made each
// thread wait S memory latencies; the whole 256 x 4096 x 4096 call with 4
// planes went 24.55 -> 24.29 us, the pass itself taking ~6 us for its 19 MB.
#include <stdint.h>

#include <algorithm>

#include "gemm_mfma.h"
#include "tmm_internal.h"

namespace tmm {
namespace {

using gemm_detail::f32x4;
using gemm_detail::out_bits;

// Adds planes [s0, s0 + G) of the quad at w onto a, in order, with all G
// loads issued first (G <= 8).
template <int G>
__device__ __forceinline__ void add_planes(f32x4 &a, const float *w, int64_t plane, int s0) {
  f32x4 b[G];
#pragma unroll
  for (int u = 0; u < G; ++u) b[u] = __builtin_nontemporal_load((const f32x4 *)(w + (s0 + u) * plane));
#pragma unroll
  for (int u = 0; u < G; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = a[e] + b[u][e];
}

// SC: the number of planes when known at compile time (2 .. 8), else 0.
template <int CT, int SC>
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
      if constexpr (SC > 0) {
        add_planes<SC - 1>(a, w, plane, 1);
      } else {
        int s = 1;
        for (; s + 8 <= S; s += 8) add_planes<8>(a, w, plane, s);
        for (; s < S; ++s) add_planes<1>(a, w, plane, s);
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
#define TMM_SPLITK_LAUNCH(SC)                                                                       \
  hipLaunchKernelGGL((splitk_reduce_kernel<CT, SC>), dim3((unsigned)blocks), dim3(256), 0, stream, W, M, N, \
                     S, (char *)C, ldc, bias, scale, vec_w, vec_c)
  switch (S) {
    case 2: TMM_SPLITK_LAUNCH(2); break;
    case 3: TMM_SPLITK_LAUNCH(3); break;
    case 4: TMM_SPLITK_LAUNCH(4); break;
    case 5: TMM_SPLITK_LAUNCH(5); break;
    case 6: TMM_SPLITK_LAUNCH(6); break;
    case 7: TMM_SPLITK_LAUNCH(7); break;
    case 8: TMM_SPLITK_LAUNCH(8); break;
    default: TMM_SPLITK_LAUNCH(0); break;
  }
#undef TMM_SPLITK_LAUNCH
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
