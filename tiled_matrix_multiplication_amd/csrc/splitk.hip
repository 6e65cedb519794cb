// Second pass of the split-K product (tmm_gemm_splitk): the S fp32 partial
// products W[s] (dense M x N planes, s = K slice) are summed in the fixed
// order W[0] + W[1] + ... + W[S-1], then scaled, the bias added and the
// result rounded once to the output format (nearest-even), as the one-pass
// epilogue does: C = scale * sum + bias, the linear-layer formula of the
// "GEMM to FlashAttention" page.
//
// HBM-bound: S*M*N*4 bytes read (the partials, each read once) and M*N
// output elements written.  A quad is 4 consecutive columns of a row: one
// 16-byte load per plane when the rows are 16-byte aligned (N % 4 == 0), an
// 8- or 16-byte store when C and its pitch allow; otherwise element by
// element with the same order of sums.  For N % 4 == 0 and S <= 8 a thread
// takes two quads and issues all 2 S loads before the first add (S a
// compile-time constant): a loop loading one plane and waiting before the
// next made each thread wait S memory latencies (the whole 256 x 4096 x
// 4096 call with 4 planes: 24.55 us that way, 24.35 with one quad per
// thread and the loads issued first, 23.9 with two).
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

template <int CT>
__device__ __forceinline__ void store_quad_out(char *dst, const float (&v)[4], bool vec, int64_t n0, int64_t N) {
  if (vec && n0 + 4 <= N) {
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

// Rows of 16-byte quads (N % 4 == 0) and a compile-time plane count SC: Q
// quads per thread (a grid stride apart), all Q SC loads issued before the
// first add.
template <int CT, int SC, int Q>
__global__ __launch_bounds__(256) void splitk_reduce_vec_kernel(const float *W, int64_t M, int64_t N, char *C,
                                                                int64_t ldc, const float *bias, float scale,
                                                                int vec_c) {
  constexpr int CE = CT == kF32 ? 4 : 2;
  const int64_t qpr = N >> 2;
  const int64_t total = M * qpr;
  const int64_t plane = M * N;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t q0 = (int64_t)blockIdx.x * 256 + threadIdx.x; q0 < total; q0 += Q * stride) {
    f32x4 b[Q][SC];
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int64_t q = q0 + i * stride;
      if (q < total) {
#pragma unroll
        for (int s = 0; s < SC; ++s) b[i][s] = __builtin_nontemporal_load((const f32x4 *)(W + s * plane + 4 * q));
      }
    }
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int64_t q = q0 + i * stride;
      if (q >= total) break;
      f32x4 a = b[i][0];
#pragma unroll
      for (int s = 1; s < SC; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = a[e] + b[i][s][e];
      const int64_t m = q / qpr, n0 = (q - m * qpr) * 4;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = a[e] * scale + (bias ? bias[n0 + e] : 0.f);
      store_quad_out<CT>(C + (m * ldc + n0) * CE, v, vec_c != 0, n0, N);
    }
  }
}

// Any S and N: 16-byte loads where a row's quad is whole and N % 4 == 0
// (planes in groups of 8), element by element elsewhere.
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
      int s = 1;
      for (; s + 8 <= S; s += 8) add_planes<8>(a, w, plane, s);
      for (; s < S; ++s) add_planes<1>(a, w, plane, s);
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
    store_quad_out<CT>(C + (m * ldc + n0) * CE, v, vec_c != 0, n0, N);
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
  if (vec_w && S >= 2 && S <= 8) {
    // two quads per thread (256 x 4096 x 4096 fp16, 4 slices: 24.35 -> 23.9 us
    // per call; four quads 24.6, eight 26.7)
    constexpr int Q = 2;
    const int64_t nb = std::min<int64_t>((quads + 256 * Q - 1) / (256 * Q), cap);
#define TMM_SPLITK_VEC(SC)                                                                               \
  hipLaunchKernelGGL((splitk_reduce_vec_kernel<CT, SC, Q>), dim3((unsigned)nb), dim3(256), 0, stream, W, M, N, \
                     (char *)C, ldc, bias, scale, vec_c)
    switch (S) {
      case 2: TMM_SPLITK_VEC(2); break;
      case 3: TMM_SPLITK_VEC(3); break;
      case 4: TMM_SPLITK_VEC(4); break;
      case 5: TMM_SPLITK_VEC(5); break;
      case 6: TMM_SPLITK_VEC(6); break;
      case 7: TMM_SPLITK_VEC(7); break;
      default: TMM_SPLITK_VEC(8); break;
    }
#undef TMM_SPLITK_VEC
    return hipGetLastError();
  }
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
