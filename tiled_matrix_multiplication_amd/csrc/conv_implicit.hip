// Fused 2-D convolution as an implicit GEMM on gfx950 matrix cores:
//
//   out = pool( act( conv(in, w) * scale[f] + bias[f] ) )
//
// the conv_fused listing of the CMU 15-418 Lecture 27 notes (section 3.1:
// NHWC input with a zero halo, weights [K][R][S][C], stride 1, per-filter
// scale and bias, ReLU, 2 x 2 max pooling, one pass), computed the way its
// section 2.3 describes implicit GEMM: the convolution is the product of
// the im2col matrix (rows = output pixels, columns = (r, s, c)) with the
// weights seen as a K x (R S C) matrix, but the im2col rows are never built
// -- each lane gathers its 16-byte pieces of them straight from the
// activation tensor, with zeros for taps outside the image.
//
// Layout of the work (fp16 / bf16 inputs, fp32 accumulation, C % 8 == 0 so
// an 8-element piece of an im2col row is 16 contiguous bytes of one pixel):
//   * GEMM rows are output pixels; with pooling they are ordered window by
//     window (4 consecutive rows = one 2 x 2 window), so the 4 accumulator
//     rows a lane holds in a v_mfma_f32_16x16x32 block are exactly one
//     pooling window of one filter and the max needs no data exchange;
//   * a workgroup computes 128 or 256 pixels x 64 filters, 4 waves of 32 or
//     64 pixels x 64 filters (2 or 4 x 4 blocks), over K-steps of 32 (r, s,
//     c) elements; operand
//     pieces are loaded into registers P steps ahead; each lane steps its own
//     (r, s, c) position forward by 32 per step;
//   * the weights are K-contiguous rows (the second operand directly);
//   * epilogue per lane: scale, bias, ReLU, max over the window, one
//     nearest-even rounding, store (NHWC output).
#include <stdint.h>

#include "conv_quad.h"
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

constexpr int kBN = 64;   // filters per workgroup
constexpr int kKS = 32;   // (r, s, c) elements per step
constexpr int kFN = 4;    // 16-filter blocks per wave
constexpr int kP = 3;     // steps of operands in flight

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
__device__ __forceinline__ uint16_t round16(float v) {
  if constexpr (F == kBF16)
    return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v, 0.f}, bf16x2)) & 0xffffu);
  else
    return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v, 0.f}, f16x2)) & 0xffffu);
}

// Position of one lane's 8-element im2col piece: tap (r, s), channel c, and
// the flat (r, s, c) index kk; advanced by 32 elements per step.
struct Tap {
  int r, s, c;
  int64_t kk;
};
__device__ __forceinline__ void advance(Tap &t, int C, int S) {
  t.kk += kKS;
  t.c += kKS;
  while (t.c >= C) {
    t.c -= C;
    if (++t.s == S) {
      t.s = 0;
      ++t.r;
    }
  }
}

// FM: 16-pixel blocks per wave (2 or 4), so a workgroup covers 64 FM pixels.
template <int AB, int CT, int FM>
__global__ __launch_bounds__(256, 2) void conv_implicit_kernel(ConvParams p) {
  constexpr int kFM = FM;
  constexpr int kBM = 64 * FM;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kq = lane >> 4;

  const int64_t P = p.H + 2 * p.pad - p.R + 1, Q = p.W + 2 * p.pad - p.S + 1;
  const int64_t OH = P / p.pool, OW = Q / p.pool;
  const int64_t Mg = p.N * P * Q;                       // GEMM rows (pixels)
  const int64_t Kg = (int64_t)p.R * p.S * p.C;          // GEMM depth (< 2^31)
  const int64_t tiles_m = (Mg + kBM - 1) / kBM;
  const int64_t bid = remap_xcd(blockIdx.x, (int64_t)gridDim.x);
  const int64_t tn = bid / tiles_m, tm = bid - tn * tiles_m;
  const int64_t m0 = tm * kBM + wave * (kBM / 4), f0 = tn * kBN;

  // Pixel (n, y, x) of each of the lane's rows (row r16 of block i); rows
  // past Mg take pixel 0 and are not stored.
  int64_t pix[kFM];   // element offset of image n's pixel (0, 0)
  int py[kFM], px[kFM];
#pragma unroll
  for (int i = 0; i < kFM; ++i) {
    int64_t m = m0 + 16 * i + r16;
    if (m >= Mg) m = 0;
    int64_t n, y, x;
    if (p.pool == 2) {
      const int64_t win = m >> 2, t = m & 3;
      n = win / (OH * OW);
      const int64_t rem = win - n * OH * OW;
      const int64_t oy = rem / OW, ox = rem - oy * OW;
      y = 2 * oy + (t >> 1);
      x = 2 * ox + (t & 1);
    } else {
      n = m / (P * Q);
      const int64_t rem = m - n * P * Q;
      y = rem / Q;
      x = rem - y * Q;
    }
    py[i] = (int)y;
    px[i] = (int)x;
    pix[i] = n * (int64_t)p.H * p.W;
  }
  // Filter rows (clamped past K).
  const uint16_t *wrow[kFN];
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int64_t f = f0 + 16 * j + r16;
    wrow[j] = (const uint16_t *)p.w + (f < p.K ? f : p.K - 1) * Kg;
  }
  const uint16_t *in = (const uint16_t *)p.in;

  f32x4 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The lane's piece: elements kk = 32 step + 8 kq .. +7.
  Tap tap;
  {
    const int k0 = 8 * kq;   // < 32
    tap.kk = k0;
    tap.c = k0 % p.C;
    const int rs = k0 / p.C;
    tap.s = rs % p.S;
    tap.r = rs / p.S;
  }
  const int64_t nsteps = (Kg + kKS - 1) / kKS;

  i32x4 fa[kP][kFM], fb[kP][kFN];
  // Taps outside the image (or past R S C) load from element 0 of the
  // tensor -- an address that is always valid -- and are then zeroed.
  auto load = [&](int slot) __attribute__((always_inline)) {
    const bool kin = tap.kk < Kg;
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      const int iy = py[i] + tap.r - p.pad, ix = px[i] + tap.s - p.pad;
      const bool ok = kin && iy >= 0 && iy < p.H && ix >= 0 && ix < p.W;
      const int64_t off = ok ? (pix[i] + (int64_t)iy * p.W + ix) * p.C + tap.c : 0;
      const i32x4 v = *(const i32x4 *)(in + off);
      fa[slot][i] = ok ? v : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const i32x4 v = *(const i32x4 *)(wrow[j] + (kin ? tap.kk : 0));
      fb[slot][j] = kin ? v : i32x4{0, 0, 0, 0};
    }
    advance(tap, p.C, p.S);
  };

#pragma unroll
  for (int q = 0; q < kP; ++q)
    if (q < nsteps) load(q);
  int64_t st = 0;
  for (; st + kP <= nsteps; st += kP) {
#pragma unroll
    for (int q = 0; q < kP; ++q) {
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] = mma<AB>(fa[q][i], fb[q][j], acc[i][j]);
      if (st + q + kP < nsteps) load(q);
    }
  }
#pragma unroll
  for (int q = 0; q < kP; ++q)
    if (st + q < nsteps) {
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] = mma<AB>(fa[q][i], fb[q][j], acc[i][j]);
    }

  // Epilogue: register t of block (i, j) is GEMM row 16 i + 4 kq + t of the
  // wave's rows, filter 16 j + r16.  With pooling the 4 rows are one window.
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int64_t f = f0 + 16 * j + r16;
    if (f >= p.K) continue;
    const float sc = p.scale ? p.scale[f] : 1.f, bi = p.bias ? p.bias[f] : 0.f;
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      const int64_t mb = m0 + 16 * i + 4 * kq;   // first of the lane's 4 rows
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[t] = acc[i][j][t] * sc + bi;
        if (p.relu) v[t] = v[t] > 0.f ? v[t] : 0.f;
      }
      if (p.pool == 2) {
        if (mb >= Mg) continue;   // the window's 4 rows exist together
        const float mx = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3]));
        const int64_t idx = (mb >> 2) * p.K + f;   // window index = pooled pixel (n, oy, ox)
        if constexpr (CT == kF32) ((float *)p.out)[idx] = mx;
        else ((uint16_t *)p.out)[idx] = round16<CT>(mx);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (mb + t >= Mg) break;
          const int64_t idx = (mb + t) * p.K + f;
          if constexpr (CT == kF32) ((float *)p.out)[idx] = v[t];
          else ((uint16_t *)p.out)[idx] = round16<CT>(v[t]);
        }
      }
    }
  }
}

// 64 pixels per wave (FM = 4: each weight piece feeds 4 pixel blocks
// instead of 2, a third fewer loads per matrix instruction) when that still
// gives two workgroups per CU; 32 otherwise.  64 x 64^2 x 64 -> 128, 3x3,
// pool: 204.8 -> 147.8 us; the 8 x 64^2 x 32 -> 64 problem (128 tiles of 256
// pixels) measured 9.8 us with 32 and 12.8 us with 64.
//
// The LDS-staged kernel of conv_quad.h takes channel counts C % 32 == 0
// (one tap per K-step) with R S C >= 96 (at least 4 steps) when its
// 128 x 128 tiles give every CU one: the listing's problem (256 tiles)
// 8.2 us against 9.9 us here.
template <int AB, int CT>
hipError_t launch_typed(const ConvParams &p, hipStream_t stream) {
  const int64_t P = p.H + 2 * p.pad - p.R + 1, Q = p.W + 2 * p.pad - p.S + 1;
  const int ov = conv_override();
  const bool quad_ok = p.C % 32 == 0 && (int64_t)p.R * p.S * p.C >= 96;
  if (quad_ok && (ov == 1 || (ov == 0 && gemm_detail::conv_quad_tiles(p) >= (int64_t)device_cu_count())))
    return gemm_detail::launch_conv_quad<AB, CT>(p, stream);
  const int64_t tn = (p.K + kBN - 1) / kBN;
  const int64_t t256 = ((p.N * P * Q + 255) / 256) * tn;
  if (t256 >= 2 * (int64_t)device_cu_count()) {
    hipLaunchKernelGGL((conv_implicit_kernel<AB, CT, 4>), dim3((unsigned)t256), dim3(256), 0, stream, p);
  } else {
    const int64_t t128 = ((p.N * P * Q + 127) / 128) * tn;
    hipLaunchKernelGGL((conv_implicit_kernel<AB, CT, 2>), dim3((unsigned)t128), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(Fmt in, Fmt out, const ConvParams &p, hipStream_t stream) {
  if (in == kBF16) return out == kF32 ? launch_typed<kBF16, kF32>(p, stream)
                                      : launch_typed<kBF16, kBF16>(p, stream);
  if (in == kF16) return out == kF32 ? launch_typed<kF16, kF32>(p, stream)
                                     : launch_typed<kF16, kF16>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace tmm
