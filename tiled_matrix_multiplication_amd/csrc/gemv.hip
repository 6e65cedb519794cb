// Matrix-vector product y = W . x (+ bias) and the K == 0 fill of the GEMM.
//
// The GEMV is the batch-1 linear layer: every weight is used once, so the
// kernel is a stream over W and its speed is HBM bandwidth, not arithmetic
// (Level-2 BLAS is memory-bound: "GEMM to FlashAttention" page, BLAS levels
// list and the batch-1 intensity case of its analyze_matmul_intensity
// listing; CMU 15-418 Lecture 27 notes, section 7, question 1: about one
// flop per weight byte).  Matrix instructions would not help; the design
// goal is enough bytes in flight:
//   * one wave (64 lanes) owns R consecutive rows (R = 1 by default, 16
//     waves per workgroup when there are enough rows); each lane issues all
//     of its 16-byte loads of those rows before using any (8 loads per row
//     for K = 4096 bf16), so a CU keeps ~128 KiB of W in flight;
//   * lane l takes chunks l, l+64, ... of a row: every load instruction of a
//     wave covers 1 KiB of contiguous weights;
//   * W is read with non-temporal loads (each byte is used once; keeping it
//     out of the caches measured 8.2 -> 7.3 us for W 4096^2 bf16 from HBM);
//   * x is loaded once per wave into registers and reused for the R rows;
//   * fp32 FMAs, then a 64-lane butterfly sum (the wave analogue of the
//     warp-shuffle reduction in the Lecture 27 fused-attention listing),
//     bias, one round-to-nearest-even store.
#include <stdio.h>
#include <stdlib.h>

#include "tmm_internal.h"

namespace tmm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int F> struct Bytes;
template <> struct Bytes<kF32> { static constexpr int value = 4; };
template <> struct Bytes<kBF16> { static constexpr int value = 2; };
template <> struct Bytes<kF16> { static constexpr int value = 2; };

__device__ __forceinline__ float lo_f16(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi_f16(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// acc += sum over the elements of a 16-byte chunk pair (w, x).
template <int F>
__device__ __forceinline__ float dot_chunk(float acc, i32x4 w, i32x4 x) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = (uint32_t)w[q], b = (uint32_t)x[q];
    if constexpr (F == kBF16) {
      acc = __builtin_fmaf(lo_bf16(a), lo_bf16(b), acc);
      acc = __builtin_fmaf(hi_bf16(a), hi_bf16(b), acc);
    } else if constexpr (F == kF16) {
      acc = __builtin_fmaf(lo_f16(a), lo_f16(b), acc);
      acc = __builtin_fmaf(hi_f16(a), hi_f16(b), acc);
    } else {
      acc = __builtin_fmaf(__uint_as_float(a), __uint_as_float(b), acc);
    }
  }
  return acc;
}

// acc += the same dot product as dot_chunk for 16-bit formats, two elements
// per instruction (v_dot2c_f32_f16 / v_dot2c_f32_bf16: both products and
// the add into the fp32 accumulator in one instruction, no conversions).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int F>
__device__ __forceinline__ float dot2_chunk(float acc, i32x4 w, i32x4 x) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // elements copied to scalars first: hipcc folds __builtin_bit_cast of a
    // vector-element lvalue to element 0
    const uint32_t a = (uint32_t)w[q], b = (uint32_t)x[q];
    if constexpr (F == kBF16)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc,
                                            false);
    else
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
  }
  return acc;
}

template <int F>
__device__ __forceinline__ float load_elem(const char *p, int64_t idx) {
  if constexpr (F == kBF16) return __uint_as_float((uint32_t)((const uint16_t *)p)[idx] << 16);
  else if constexpr (F == kF16) return (float)((const _Float16 *)p)[idx];
  else return ((const float *)p)[idx];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int YT>
__device__ __forceinline__ void put(void *y, int64_t i, float v) {
  if constexpr (YT == kF32) ((float *)y)[i] = v;
  else if constexpr (YT == kBF16) ((uint16_t *)y)[i] = to_bf16(v);
  else ((uint16_t *)y)[i] = __builtin_bit_cast(uint16_t, (_Float16)v);
}

constexpr int kWaves = 4;  // waves per workgroup of the element path
constexpr int kUnroll = 8; // 16-byte chunks per lane per row in one pass

// 16-byte path: K*E is a multiple of 16 and W, x, ldw are 16-byte aligned.
// WPB waves per workgroup, R rows per wave.  WHOLE: the row is a whole
// number of passes (K*E a multiple of 64 lanes x kUnroll x 16 bytes, e.g.
// K = 4096 bf16), so no load needs a bound check; the predicated form
// measured 0.3-0.4 us slower per 4096 x 4096 launch, where the loads'
// issue at the start of the kernel is on the critical path.
template <int WT, int YT, int R, int WPB, bool WHOLE>
__global__ __launch_bounds__(64 * WPB) void gemv_vec_kernel(GemvParams p) {
  constexpr int E = Bytes<WT>::value;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * WPB + (threadIdx.x >> 6)) * R;
  if (row0 >= p.N) return;
  const int64_t nchunks = p.K * E / 16;
  const char *W = (const char *)p.W;
  const char *x = (const char *)p.x;
  const char *wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rr = row0 + r < p.N ? row0 + r : p.N - 1;
    wrow[r] = W + rr * p.ldw * E;
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;

  for (int64_t c0 = 0; c0 < nchunks; c0 += 64 * kUnroll) {
    i32x4 xv[kUnroll], wv[R][kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t cc = c0 + u * 64 + lane;
      const bool ok = WHOLE || cc < nchunks;
#pragma unroll
      for (int r = 0; r < R; ++r)
        wv[r][u] = ok ? __builtin_nontemporal_load((const i32x4 *)(wrow[r] + cc * 16))
                      : i32x4{0, 0, 0, 0};
      xv[u] = ok ? *(const i32x4 *)(x + cc * 16) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = dot_chunk<WT>(acc[r], wv[r][u], xv[u]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float s = wave_sum(acc[r]);
    if (lane == r && row0 + r < p.N) put<YT>(p.y, row0 + r, s + (p.bias ? p.bias[row0 + r] : 0.f));
  }
}

// Few rows at once, Y[m] = W . X[m] (+ bias) for m < MV <= 8 (batched
// decode through one linear layer): the weight stream of the GEMV above with
// MV dot products per weight chunk, two elements per dot instruction (with
// conversions and one FMA per element, M = 4 was VALU-bound: 10.2 us
// against 9.2 us for the skinny MFMA kernel).  The workgroup stages the MV rows of X
// for one pass (64 lanes x kUnroll chunks = 8 KiB of each row) in LDS, so X
// is read from L2 once per workgroup instead of once per wave, and each lane
// reads its chunks of the MV rows back 16 bytes at a time (consecutive lanes,
// consecutive chunks).  A wave's weight loads for the pass are issued before
// the staging barrier.  Rows past N read the last row and are not stored;
// chunks past K are zero (K*E a multiple of 16).
template <int WT, int YT, int MV, int R, int WPB>
__global__ __launch_bounds__(64 * WPB) void gemv_multi_kernel(GemvMParams p) {
  constexpr int E = Bytes<WT>::value;
  constexpr int PASS = 64 * kUnroll;                 // chunks of a row per pass
  constexpr int XPT = (MV * PASS + 64 * WPB - 1) / (64 * WPB);  // X chunks staged per thread
  __shared__ __attribute__((aligned(16))) i32x4 xs[MV][PASS];
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * WPB + (threadIdx.x >> 6)) * R;
  const int64_t nchunks = p.K * E / 16;
  const char *wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rr = row0 + r < p.N ? row0 + r : p.N - 1;
    wrow[r] = (const char *)p.W + rr * p.ldw * E;
  }
  float acc[R][MV];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MV; ++m) acc[r][m] = 0.f;

  for (int64_t c0 = 0; c0 < nchunks; c0 += PASS) {
    // X of the pass is loaded first, so that waiting for it (to write it to
    // LDS) does not wait for the weight loads issued after it; then the
    // weight rows in order, so row r's products start while the later rows
    // are still arriving.
    i32x4 xv[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int t = (int)threadIdx.x + i * 64 * WPB;
      const int m = t / PASS, c = t - m * PASS;
      const int64_t cc = c0 + c;
      xv[i] = (t < MV * PASS && cc < nchunks)
                  ? *(const i32x4 *)((const char *)p.x + (m * p.ldx * E + cc * 16))
                  : i32x4{0, 0, 0, 0};
    }
    i32x4 wv[R][kUnroll];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t cc = c0 + u * 64 + lane;
        wv[r][u] = cc < nchunks ? __builtin_nontemporal_load((const i32x4 *)(wrow[r] + cc * 16))
                                : i32x4{0, 0, 0, 0};
      }
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int t = (int)threadIdx.x + i * 64 * WPB;
      if (t < MV * PASS) xs[t / PASS][t % PASS] = xv[i];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int m = 0; m < MV; ++m) acc[r][m] = dot2_chunk<WT>(acc[r][m], wv[r][u], xs[m][u * 64 + lane]);
    __syncthreads();   // the pass's X is read before the next pass overwrites it
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
    const float b = (p.bias && row < p.N) ? p.bias[row] : 0.f;
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      const float s = wave_sum(acc[r][m]);
      if (lane == m && row < p.N) put<YT>(p.y, m * p.ldy + row, s + b);
    }
  }
}

// Element path for any alignment.
template <int WT, int YT>
__global__ __launch_bounds__(64 * kWaves) void gemv_elem_kernel(GemvParams p) {
  constexpr int E = Bytes<WT>::value;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= p.N) return;
  const char *w = (const char *)p.W + row * p.ldw * E;
  float acc = 0.f;
  for (int64_t k = lane; k < p.K; k += 64)
    acc = __builtin_fmaf(load_elem<WT>(w, k), load_elem<WT>((const char *)p.x, k), acc);
  const float s = wave_sum(acc);
  if (lane == 0) put<YT>(p.y, row, s + (p.bias ? p.bias[row] : 0.f));
}

template <int WT, int YT, int R, int WPB>
void launch_vec(const GemvParams &p, hipStream_t stream) {
  const int64_t waves = (p.N + R - 1) / R;
  const unsigned blocks = (unsigned)((waves + WPB - 1) / WPB);
  const bool whole = (p.K * Bytes<WT>::value) % (64 * kUnroll * 16) == 0;
  if (whole)
    hipLaunchKernelGGL((gemv_vec_kernel<WT, YT, R, WPB, true>), dim3(blocks), dim3(64 * WPB), 0, stream, p);
  else
    hipLaunchKernelGGL((gemv_vec_kernel<WT, YT, R, WPB, false>), dim3(blocks), dim3(64 * WPB), 0, stream, p);
}

// Rows per wave and waves per workgroup of the 16-byte path: R * 100 + W
// from the library's override ("gemv=<R>x<W>", R in {1, 2, 4}, W in
// {4, 8, 16}), 0 for the automatic choice.
int gemv_cfg() { return gemv_override(); }

template <int WT, int YT>
hipError_t launch_typed(bool vec, const GemvParams &p, hipStream_t stream) {
  if (vec) {
    switch (gemv_cfg()) {
      case 104: launch_vec<WT, YT, 1, 4>(p, stream); break;
      case 108: launch_vec<WT, YT, 1, 8>(p, stream); break;
      case 116: launch_vec<WT, YT, 1, 16>(p, stream); break;
      case 204: launch_vec<WT, YT, 2, 4>(p, stream); break;
      case 208: launch_vec<WT, YT, 2, 8>(p, stream); break;
      case 216: launch_vec<WT, YT, 2, 16>(p, stream); break;
      case 404: launch_vec<WT, YT, 4, 4>(p, stream); break;
      case 408: launch_vec<WT, YT, 4, 8>(p, stream); break;
      case 416: launch_vec<WT, YT, 4, 16>(p, stream); break;
      default:
        // One row per wave; sixteen waves per workgroup once that still
        // gives every CU a workgroup (W 4096 x 4096 bf16: 6.87 against
        // 7.01 us per launch for four), four below (more CUs streaming).
        if (p.N >= 16 * (int64_t)device_cu_count()) launch_vec<WT, YT, 1, 16>(p, stream);
        else launch_vec<WT, YT, 1, 4>(p, stream);
        break;
    }
  } else {
    const unsigned blocks = (unsigned)((p.N + kWaves - 1) / kWaves);
    hipLaunchKernelGGL((gemv_elem_kernel<WT, YT>), dim3(blocks), dim3(64 * kWaves), 0, stream, p);
  }
  return hipGetLastError();
}

// Value of a stored output element (the old C of the full form).
template <int CT>
__device__ __forceinline__ float get(const void *C, int64_t idx) {
  if constexpr (CT == kF32) return ((const float *)C)[idx];
  else if constexpr (CT == kBF16) return __uint_as_float((uint32_t)((const uint16_t *)C)[idx] << 16);
  else return (float)__builtin_bit_cast(_Float16, ((const uint16_t *)C)[idx]);
}

// ---- K == 0 fill for the GEMM: C = act(bias + beta * old C), the empty
// sum (bias and beta default to none: C = 0)
template <int CT>
__global__ __launch_bounds__(256) void fill_kernel(GemmParams p) {
  const int64_t per = p.M * p.N;
  const int64_t total = per * p.batch;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t z = t / per;
    const int64_t rem = t - z * per;
    const int64_t row = rem / p.N, col = rem - row * p.N;
    float v = p.bias ? p.bias[col] : 0.f;
    const int64_t idx = z * p.strideC + row * p.ldc + col;
    if (p.beta != 0.f) v += p.beta * get<CT>(p.C, idx);
    if (p.act == 1) v = v > 0.f ? v : 0.f;
    put<CT>(p.C, idx, v);
  }
}

}  // namespace

hipError_t launch_gemv(Fmt w, Fmt y, bool vec, const GemvParams &p, hipStream_t stream) {
  if (w == kF32) return launch_typed<kF32, kF32>(vec, p, stream);
  if (w == kBF16)
    return y == kF32 ? launch_typed<kBF16, kF32>(vec, p, stream)
                     : launch_typed<kBF16, kBF16>(vec, p, stream);
  if (w == kF16)
    return y == kF32 ? launch_typed<kF16, kF32>(vec, p, stream)
                     : launch_typed<kF16, kF16>(vec, p, stream);
  return hipErrorInvalidValue;
}

namespace {
// One row per wave, sixteen waves per workgroup: two rows per wave (the
// second row's weights arriving under the first row's products) and eight
// waves per workgroup measured slower (M = 4: 10.2 and 9.4 against 9.0 us).
template <int WT, int YT, int MV>
hipError_t launch_multi_mv(const GemvMParams &p, hipStream_t stream) {
  constexpr int R = 1, WPB = 16;
  const unsigned blocks = (unsigned)((p.N + R * WPB - 1) / (R * WPB));
  hipLaunchKernelGGL((gemv_multi_kernel<WT, YT, MV, R, WPB>), dim3(blocks), dim3(64 * WPB), 0, stream, p);
  return hipGetLastError();
}

template <int WT, int YT>
hipError_t launch_multi_typed(const GemvMParams &p, hipStream_t stream) {
  switch (p.M) {
    case 2: return launch_multi_mv<WT, YT, 2>(p, stream);
    case 3: return launch_multi_mv<WT, YT, 3>(p, stream);
    case 4: return launch_multi_mv<WT, YT, 4>(p, stream);
    case 5: return launch_multi_mv<WT, YT, 5>(p, stream);
    case 6: return launch_multi_mv<WT, YT, 6>(p, stream);
    case 7: return launch_multi_mv<WT, YT, 7>(p, stream);
    case 8: return launch_multi_mv<WT, YT, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_gemv_multi(Fmt w, Fmt y, const GemvMParams &p, hipStream_t stream) {
  if (w == kBF16)
    return y == kF32 ? launch_multi_typed<kBF16, kF32>(p, stream)
                     : launch_multi_typed<kBF16, kBF16>(p, stream);
  if (w == kF16)
    return y == kF32 ? launch_multi_typed<kF16, kF32>(p, stream)
                     : launch_multi_typed<kF16, kF16>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fill(Fmt c, const GemmParams &p, hipStream_t stream) {
  const int64_t total = p.M * p.N * p.batch;
  const int64_t want = (total + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? (want > 0 ? want : 1) : 65536);
  switch (c) {
    case kF32: hipLaunchKernelGGL(fill_kernel<kF32>, dim3(blocks), dim3(256), 0, stream, p); break;
    case kBF16: hipLaunchKernelGGL(fill_kernel<kBF16>, dim3(blocks), dim3(256), 0, stream, p); break;
    case kF16: hipLaunchKernelGGL(fill_kernel<kF16>, dim3(blocks), dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tmm
