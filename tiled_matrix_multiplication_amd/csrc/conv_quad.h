// Fused 2-D convolution as an implicit GEMM on the four-wave LDS ring:
//
//   out = pool( act( conv(in, w) * scale[f] + bias[f] ) )
//
// the operation of conv_implicit.hip (the conv_fused listing of the CMU
// 15-418 Lecture 27 notes, section 3.1; implicit GEMM as its section 2.3
// describes it: rows = output pixels, columns = (r, s, c) taps, the weights
// a K x (R S C) matrix), for channel counts C that are multiples of 32.
// There the operands went straight from global memory to registers, every
// wave loading its own filter pieces; here a workgroup stages both operands
// in LDS, as the four-wave GEMM does (gemm_quad.h), so every piece is
// fetched once per workgroup and read by two waves:
//   * a workgroup computes 128 pixels x 128 filters, four waves of 64 x 64
//     (4 x 4 blocks of v_mfma_f32_16x16x32), in K-steps of 32 (r, s, c)
//     elements; with C % 32 == 0 one step lies within one tap (r, s) and
//     covers channels 32 cb .. 32 cb + 31.  Its four stages take 64 KiB of
//     LDS, so two workgroups share a CU and one's prologue and epilogue
//     (a 3 x 3 tap over 64 channels is only 18 steps) overlap the other's
//     matrix work: 64 x 64^2 x 64 -> 128, 3 x 3, pooled, 59.3 us against
//     73.3 us with one workgroup of 256 x 128 per CU;
//   * the im2col rows are never built: a stage row is one output pixel's 64
//     bytes of the step, filled by direct 16-byte global->LDS loads whose
//     per-lane source is the pixel's tap neighbour (y + r - pad,
//     x + s - pad), or a 16-byte block of zeros for taps outside the image;
//     the weights are K-contiguous rows, loaded as the GEMM loads a
//     K-contiguous B;
//   * the ring, the swizzle, the fragment reads and the step schedule are
//     those of gemm_quad.h (loads three steps ahead, one
//     barrier per step, next step's fragments read during the current one);
//     R S C / 32 steps are padded to an even count with all-zero steps;
//   * with pooling the GEMM rows are ordered window by window (4
//     consecutive rows = one 2 x 2 window), so the 4 accumulator rows a lane
//     holds in a 16x16 block are one window of one filter: the epilogue
//     applies scale, bias and ReLU, takes the max of the 4 and rounds once.
#pragma once

#include <type_traits>

#include "gemm_quad.h"

namespace tmm {
namespace gemm_detail {

// Source of the direct loads for taps outside the image and for the steps
// past R S C.
__device__ __attribute__((aligned(64))) const uint32_t kConvZeros[16] = {0u};

// Pixel (image n, row y, column x) of GEMM row m: raster order, or window by
// window when pooling 2 x 2 (OH x OW windows per image).
__device__ __forceinline__ void conv_pixel(int64_t m, int pool, int64_t P, int64_t Q, int64_t OH, int64_t OW,
                                           int64_t &n, int &y, int &x) {
  if (pool == 2) {
    const int64_t win = m >> 2, t = m & 3;
    n = win / (OH * OW);
    const int64_t rem = win - n * OH * OW;
    const int64_t oy = rem / OW, ox = rem - oy * OW;
    y = (int)(2 * oy + (t >> 1));
    x = (int)(2 * ox + (t & 1));
  } else {
    n = m / (P * Q);
    const int64_t rem = m - n * P * Q;
    y = (int)(rem / Q);
    x = (int)(rem - (int64_t)y * Q);
  }
}

template <int AB, int CT>
__global__ __launch_bounds__(256, 2) void conv_quad_kernel(ConvParams p) {
  constexpr int BM = 128, BN = 128, NW = 4;
  constexpr int WTM = BM / 2, WTN = BN / 2;    // each wave's block
  constexpr int FM = WTM / 16, FN = WTN / 16;  // 4 x 4 accumulators
  constexpr int ROWB = kRingRowBytes;          // 64 bytes of a step per row
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int S = kRingStages;               // 4
  constexpr int LA = A_BYTES / 1024 / NW;      // direct loads per wave per step: 2 (pixels)
  constexpr int LB = B_BYTES / 1024 / NW;      // 2 (filters)
  constexpr int LPS = LA + LB;
  static_assert(LPS <= FM, "one direct load per row block at most");
  // slots (instruction index within a row block) of the B read and the load
  constexpr int QB0 = 1, QD = 2;

  __shared__ __attribute__((aligned(16))) char lds[S * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int H = p.H, W = p.W, C = p.C, R = p.R, SW = p.S, pad = p.pad;
  const int64_t P = H + 2 * pad - R + 1, Q = W + 2 * pad - SW + 1;
  const int64_t OH = P / p.pool, OW = Q / p.pool;
  const int64_t Mg = p.N * P * Q;                 // GEMM rows (pixels)
  const int64_t Kg = (int64_t)R * SW * C;         // GEMM depth
  const int64_t KF = p.K;                         // filters
  const int64_t tiles_m = (Mg + BM - 1) / BM, tiles_n = (KF + BN - 1) / BN;
  int64_t tm, tn;
  group_order(remap_xcd(blockIdx.x, (int64_t)gridDim.x), tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const char *in = (const char *)p.in;
  const char *zeros = (const char *)kConvZeros;

  // ---- direct-load sources.  Load q of wave w fills stage rows
  // w BM/4 + 16 q .. +15 (A) or w BN/4 + 16 q (B); lane L lands at row
  // L / 4, position L % 4 and loads logical chunk (L % 4) ^ qswz64(row).
  // A: the lane's pixel (rows past Mg take the last pixel; not stored).
  int64_t a_pix[LA];   // byte offset of pixel (n, y, x), channel 0, plus the chunk
  int a_y[LA], a_x[LA];
#pragma unroll
  for (int q = 0; q < LA; ++q) {
    const int row = wave * (BM / NW) + q * 16 + (lane >> 2);
    int64_t n;
    int y, x;
    conv_pixel(min64(m0 + row, Mg - 1), p.pool, P, Q, OH, OW, n, y, x);
    a_y[q] = y;
    a_x[q] = x;
    a_pix[q] = ((n * H + y) * W + x) * C * 2 + (((lane & 3) ^ qswz64(row)) << 4);
  }
  // B: filter rows (past K: the last filter; not stored).
  const char *b_row[LB];
#pragma unroll
  for (int q = 0; q < LB; ++q) {
    const int row = wave * (BN / NW) + q * 16 + (lane >> 2);
    const int64_t f = min64(n0 + row, KF - 1);
    b_row[q] = (const char *)p.w + f * Kg * 2 + (((lane & 3) ^ qswz64(row)) << 4);
  }
  const uint32_t lds0 = lds_addr(lds);

  // Tap of the next step to load: channel block cb (32 channels), tap
  // (r, s); steps with r == R are the zero padding.  Advanced once per step.
  const int cblocks = C / 32;
  int ld_cb = 0, ld_r = 0, ld_s = 0;
  int64_t ld_k = 0;   // byte offset of the step in a filter row
  struct StepSrc {
    int dy, dx;       // tap offset from the output pixel
    int64_t off;      // byte offset of the tap's channel block from the pixel
    bool live;        // a step within R S C
    int64_t koff;
  };
  auto step_src = [&]() __attribute__((always_inline)) {
    StepSrc t;
    t.dy = ld_r - pad;
    t.dx = ld_s - pad;
    t.off = ((int64_t)t.dy * W + t.dx) * C * 2 + (int64_t)ld_cb * 64;
    t.live = ld_r < R;
    t.koff = ld_k;
    return t;
  };
  auto advance = [&]() __attribute__((always_inline)) {
    const int cb1 = ld_cb + 1;
    const bool wrap_c = cb1 == cblocks;
    ld_cb = wrap_c ? 0 : cb1;
    const int s1 = ld_s + (wrap_c ? 1 : 0);
    const bool wrap_s = s1 == SW;
    ld_s = wrap_s ? 0 : s1;
    ld_r += wrap_s ? 1 : 0;
    ld_k += ROWB;
  };
  auto issue_one = [&](const StepSrc &t, int stage, int q) __attribute__((always_inline)) {
    const uint32_t la = lds0 + (uint32_t)(stage * STAGE);
    if (q < LA) {
      const bool ok = t.live && (unsigned)(a_y[q] + t.dy) < (unsigned)H && (unsigned)(a_x[q] + t.dx) < (unsigned)W;
      dma16(ok ? in + a_pix[q] + t.off : zeros, la + (wave * (BM / NW) + q * 16) * ROWB);
    } else {
      const int i = q - LA;
      dma16(t.live ? b_row[i] + t.koff : zeros, la + A_BYTES + (wave * (BN / NW) + i * 16) * ROWB);
    }
  };

  // ---- fragment addresses (bytes within a stage): row block base + lane
  // row l16, chunk G (swizzled)
  const int l16 = lane & 15, G = lane >> 4;
  const int a_lane = l16 * ROWB + ((G ^ qswz64(l16)) << 4);
  const int a_base = wm * WTM * ROWB + a_lane;                   // + 1024 i
  const int b_base = A_BYTES + wn * WTN * ROWB + a_lane;         // + 1024 j

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  i32x4 fa[FM];
  i32x4 fb0[FN], fb1[FN];
  auto read_a = [&](int stage, int i) __attribute__((always_inline)) {
    fa[i] = *(const i32x4 *)(lds + stage * STAGE + a_base + i * 16 * ROWB);
  };
  auto read_b = [&](int stage, i32x4 (&fb)[FN], int j) __attribute__((always_inline)) {
    fb[j] = *(const i32x4 *)(lds + stage * STAGE + b_base + j * 16 * ROWB);
  };

  const int64_t nsteps = ((Kg / 32 + 1) / 2) * 2;   // even, >= 4 (checked by the host)
  constexpr int D = S - 1;                           // steps loaded ahead
  auto stage_of = [](int64_t k) { return (int)(k & (S - 1)); };
#pragma unroll
  for (int k = 0; k < D; ++k) {
    const StepSrc t = step_src();
#pragma unroll
    for (int q = 0; q < LPS; ++q) issue_one(t, k, q);
    advance();
  }
  // steps 0 and 1 landed (step 2 may still be in flight), then published
  __builtin_amdgcn_s_waitcnt(vm_wait(LPS));
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) read_a(0, i);
#pragma unroll
  for (int j = 0; j < FN; ++j) read_b(0, fb0, j);

  // Step kt, as in gemm_quad.h: matrix instructions from fa / cb, the next
  // step's fragments into fa (row block by row block) and nb (fragment i in
  // row block i), step kt + 3's direct loads (load q in row block q) into
  // the stage step kt - 1 used, then the barrier that publishes step kt + 2.
  auto step = [&](int64_t kt, const i32x4 (&cb)[FN], i32x4 (&nb)[FN], auto load_tag)
      __attribute__((always_inline)) {
    constexpr bool LOAD = decltype(load_tag)::value;
    const int nxt = stage_of(kt + 1);
    const int lst = stage_of(kt + D);
    StepSrc t;
    if constexpr (LOAD) t = step_src();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[i][j] = mma16<AB>(fa[i], cb[j], acc[i][j]);
        if (i < FN && j == QB0) read_b(nxt, nb, i);
        if (LOAD && i < LPS && j == QD) issue_one(t, lst, i);
        __builtin_amdgcn_sched_barrier(0);
      }
      read_a(nxt, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (LOAD) advance();
    __builtin_amdgcn_s_waitcnt(vm_only_wait(LOAD ? LPS : 0));
    __builtin_amdgcn_s_barrier();
  };
  using Load = std::integral_constant<bool, true>;
  using NoLoad = std::integral_constant<bool, false>;
  int64_t kt = 0;
  for (; kt + 4 < nsteps; kt += 2) {
    step(kt, fb0, fb1, Load());
    step(kt + 1, fb1, fb0, Load());
  }
  step(kt, fb0, fb1, Load());
  step(kt + 1, fb1, fb0, NoLoad());
  step(kt + 2, fb0, fb1, NoLoad());
  step(kt + 3, fb1, fb0, NoLoad());

  // ---- epilogue: register t of block (i, j) is GEMM row 16 i + 4 G + t of
  // the wave's rows, filter 16 j + l16; with pooling the 4 rows are a window.
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t f = n0 + wn * WTN + 16 * j + l16;
    if (f >= KF) continue;
    const float sc = p.scale ? p.scale[f] : 1.f, bi = p.bias ? p.bias[f] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t mb = m0 + wm * WTM + 16 * i + 4 * G;   // first of the lane's 4 rows
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[t] = acc[i][j][t] * sc + bi;
        if (p.relu) v[t] = v[t] > 0.f ? v[t] : 0.f;
      }
      if (p.pool == 2) {
        if (mb >= Mg) continue;   // the window's 4 rows exist together
        const float mx = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3]));
        store_out<CT>((char *)p.out, (mb >> 2) * KF + f, mx);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (mb + t >= Mg) break;
          store_out<CT>((char *)p.out, (mb + t) * KF + f, v[t]);
        }
      }
    }
  }
}

// Workgroups of the LDS-staged kernel for a problem.
inline int64_t conv_quad_tiles(const ConvParams &p) {
  const int64_t P = p.H + 2 * p.pad - p.R + 1, Q = p.W + 2 * p.pad - p.S + 1;
  return ((p.N * P * Q + 127) / 128) * ((p.K + 127) / 128);
}

// The host has checked C % 32 == 0 and R S C >= 96.
template <int AB, int CT>
hipError_t launch_conv_quad(const ConvParams &p, hipStream_t stream) {
  hipLaunchKernelGGL((conv_quad_kernel<AB, CT>), dim3((unsigned)conv_quad_tiles(p)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gemm_detail
}  // namespace tmm
