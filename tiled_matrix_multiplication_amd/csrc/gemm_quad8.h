// Tiled GEMM on gfx950 matrix cores for fp8 (OCP E4M3) inputs with four
// waves per 256x256 tile, each wave owning a 128x128 block of C:
//
//   C[z] = scale * A[z] . op(B[z]) (+ bias),  row-major, z < batch
//
// for K a multiple of 128 (at least 256) and 16-byte-whole operand chunks.
// It is the four-wave kernel of gemm_quad.h on the fp8 instruction: the
// same four-stage LDS ring of 64-byte K-steps (64 fp8 per tile row), the
// same direct 16-byte global->LDS loads three steps ahead and the same
// barrier-per-step protocol; a wave's block is 4x4 accumulators of
// v_mfma_f32_32x32x64_f8f6f4 (256 fp32 accumulators per lane in the AGPRs),
// against the eight 128x64 waves of the ring kernel: each A block is read
// by two waves instead of four, so a step reads a third less from LDS (the
// register blocking of the Lecture 27 notes, section 2.4, with the
// low-precision inputs and fp32 accumulation of section 2.7).
// Fragments (as in the ring kernel's fp8 path, so that A and B pair the
// same k): lane l of a 32x32x64 block holds row / column l % 32 and the
// 16-byte chunks g and 2 + g (g = l / 32) of the 64-byte K-step --
//   * A and a K-contiguous B: two 16-byte reads of the stage's 64-byte rows
//     (chunk c of row r at c ^ ((r >> 2) & 3));
//   * an N-contiguous B: the stage holds k-rows of 256 fp8 as in memory,
//     chunk c of k-row r at c ^ 2 (r mod 8), read with ds_read_b64_tr_b8
//     (lane i of a 16-lane group receives 8 consecutive k of column i when
//     lane s points at k-row k0 + s / 2, columns n0 + 8 (s mod 2) .. +7):
//     four such reads, pieces t = 0..3 holding k 32 (t / 2) + 16 g + 8 (t mod
//     2) .. +7, make the 32 bytes that pair with A's.
// Within a step a wave issues its 16 matrix instructions row block by row
// block; between them the next step's B fragment of that row block (four
// transposing or two plain reads), two of its eight direct loads, and after
// the row block the next step's A fragment of that row block into the same
// registers.
#pragma once

#include <type_traits>

#include "gemm_mfma.h"
#include "gemm_quad.h"
#include "gemm_ring.h"

namespace tmm {
namespace gemm_detail {

template <int CT, bool NT>
__global__ __launch_bounds__(256) void gemm_quad8_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256, NW = 4;
  constexpr int WTM = BM / 2, WTN = BN / 2;     // each wave's 128x128 block of C
  constexpr int FM = WTM / 32, FN = WTN / 32;   // 4x4 accumulators of 32x32
  constexpr int CE = FmtBytes<CT>::value;
  constexpr int ROWB = kRingRowBytes;           // 64 bytes = 64 fp8 of K per tile row per step
  constexpr int BK = ROWB;
  constexpr int A_BYTES = BM * ROWB;            // 16 KiB
  constexpr int B_BYTES = BN * ROWB;            // 16 KiB
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int S = kRingStages;                // 4
  constexpr int NB_ROW = BN;                    // NN: bytes of one k-row of the B stage
  constexpr int CPR = NB_ROW / 16, RPI = 64 / CPR;  // NN: 16 chunks per k-row, 4 k-rows per load
  constexpr int LA = A_BYTES / 1024 / NW;       // 4 direct loads per wave per step (A)
  constexpr int LB = B_BYTES / 1024 / NW;       // 4 (B)
  constexpr int LPS = LA + LB;
  static_assert(S == 4 && LPS == 2 * FM, "geometry");

  __shared__ __attribute__((aligned(16))) char lds[S * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, l32 = lane & 31;
  const int G = lane >> 4, q = lane & 15;

  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  int64_t pid = remap_xcd(blockIdx.x, (int64_t)gridDim.x);
  const int64_t z = pid / tiles;
  pid -= z * tiles;
  int64_t tm, tn;
  group_order(pid, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const char *A = (const char *)p.A + z * p.strideA;
  const char *B = (const char *)p.B + z * p.strideB;

  // ---- direct-load sources (byte offsets < 4 GiB, checked by the host);
  // layout as in gemm_quad.h, with the fp8 NN swizzle nn_swz<1>.
  uint32_t a_off[LA], b_off[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int row = wave * (BM / NW) + i * 16 + (lane >> 2);
    const int64_t r = min64(m0 + row, M - 1);
    a_off[i] = (uint32_t)(r * p.lda + (((lane & 3) ^ swz64(row)) << 4));
  }
  if constexpr (NT) {
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = wave * (BN / NW) + i * 16 + (lane >> 2);
      const int64_t r = min64(n0 + row, N - 1);
      b_off[i] = (uint32_t)(r * p.ldb + (((lane & 3) ^ swz64(row)) << 4));
    }
  } else {
    // instruction i of wave w fills k-rows 16 w + 4 i .. +3; lane L lands at
    // k-row L / 16, position L % 16 and loads logical chunk (L % 16) ^
    // nn_swz<1>(row); a chunk wholly past N (the host ensures N % 16 == 0)
    // reads chunk 0 of the tile and only feeds outputs that are not stored.
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = wave * (BK / NW) + i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ nn_swz<1>(row);
      const int64_t col = n0 + (int64_t)c * 16;
      const int64_t ccol = col < N ? col : n0;
      b_off[i] = (uint32_t)((int64_t)row * p.ldb + ccol);
    }
  }
  const int64_t kstep_b = NT ? (int64_t)ROWB : (int64_t)BK * p.ldb;
  const uint32_t lds0 = lds_addr(lds);

  // ---- fragment addresses (bytes within a stage).  Block bases are
  // multiples of 32 rows, so swz64(base + l32) = swz64(l32).
  const int a_c0 = ((g ^ swz64(l32)) << 4), a_c1 = (((2 + g) ^ swz64(l32)) << 4);
  const int a_row = (wm * WTM + l32) * ROWB;                    // + 2048 i
  const int bt_row = A_BYTES + (wn * WTN + l32) * ROWB;         // NT: + 2048 j

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  i32x8 fa[FM];
  i32x8 fb0[FN], fb1[FN];

  auto issue_one = [&](int64_t kt, int stage, int qq) __attribute__((always_inline)) {
    const uint32_t la = lds0 + (uint32_t)(stage * STAGE);
    if (qq < LA) {
      dma16(A + kt * ROWB + a_off[qq], la + (wave * (BM / NW) + qq * 16) * ROWB);
    } else {
      const int i = qq - LA;
      if constexpr (NT)
        dma16(B + kt * kstep_b + b_off[i], la + A_BYTES + (wave * (BN / NW) + i * 16) * ROWB);
      else
        dma16(B + kt * kstep_b + b_off[i], la + A_BYTES + (wave * (BK / NW) + i * RPI) * NB_ROW);
    }
  };
  auto read_a = [&](int stage, int i) __attribute__((always_inline)) {
    const char *base = lds + stage * STAGE + a_row + i * 32 * ROWB;
    const i32x4 lo = *(const i32x4 *)(base + a_c0), hi = *(const i32x4 *)(base + a_c1);
    fa[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // The next step's B fragment j in two halves h (NN: pieces 2h, 2h + 1;
  // NT: one 16-byte read each).
  i32x2 piece[FN][2];
  auto read_b = [&](int stage, i32x8 (&fb)[FN], int j, int h) __attribute__((always_inline)) {
    const char *base = lds + stage * STAGE;
    if constexpr (NT) {
      const i32x4 v = *(const i32x4 *)(base + bt_row + j * 32 * ROWB + (h ? a_c1 : a_c0));
      if (h == 0) {
        piece[j][0] = i32x2{v[0], v[1]};
        piece[j][1] = i32x2{v[2], v[3]};
      } else {
        fb[j] = i32x8{piece[j][0][0], piece[j][0][1], piece[j][1][0], piece[j][1][1], v[0], v[1], v[2], v[3]};
      }
    } else {
      i32x2 pc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = 2 * h + u;
        const int row = 32 * (t >> 1) + 16 * g + 8 * (t & 1) + (q >> 1);
        const int chunk = (wn * WTN + j * 32) / 16 + (G & 1);
        pc[u] = lds_read_tr8(base + A_BYTES + row * NB_ROW + ((chunk ^ nn_swz<1>(row)) << 4) + 8 * (q & 1));
      }
      if (h == 0) {
        piece[j][0] = pc[0];
        piece[j][1] = pc[1];
      } else {
        fb[j] = i32x8{piece[j][0][0], piece[j][0][1], piece[j][1][0], piece[j][1][1], pc[0][0], pc[0][1],
                      pc[1][0], pc[1][1]};
      }
    }
  };

  const int64_t nsteps = K / BK;  // the host guarantees K % (2 BK) == 0, K >= 4 BK
  constexpr int D = S - 1;        // steps loaded ahead
  auto stage_of = [](int64_t k) { return (int)(k & (S - 1)); };
  for (int64_t k = 0; k < D; ++k)
#pragma unroll
    for (int qq = 0; qq < LPS; ++qq) issue_one(k, (int)k, qq);
  // steps 0 and 1 landed (step 2 may still be in flight), then published
  __builtin_amdgcn_s_waitcnt(vm_wait(LPS));
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) read_a(0, i);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    read_b(0, fb0, j, 0);
    read_b(0, fb0, j, 1);
  }

  // Step kt, as in gemm_quad.h: matrix instructions from fa / cb; the next
  // step's B fragment i during row block i (into nb) and A fragment i after
  // it (into fa); with LOAD, loads 2i and 2i + 1 of step kt + 3 during row
  // block i into the stage step kt - 1 used; the barrier then publishes step
  // kt + 2.  The last three steps are written out after the loop.
  auto step = [&](int64_t kt, const i32x8 (&cb)[FN], i32x8 (&nb)[FN], auto load_tag)
      __attribute__((always_inline)) {
    constexpr bool LOAD = decltype(load_tag)::value;
    const int nxt = stage_of(kt + 1);
    const int lst = stage_of(kt + D);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        // format code 0 (fp8 E4M3) for both operands; zero scale operands
        // select the unscaled instruction
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], cb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        if (j == 0) read_b(nxt, nb, i, 0);
        if (j == 1) read_b(nxt, nb, i, 1);
        if (LOAD && j == 2) issue_one(kt + D, lst, 2 * i);
        if (LOAD && j == 3) issue_one(kt + D, lst, 2 * i + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      read_a(nxt, i);
      __builtin_amdgcn_sched_barrier(0);
    }
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

  // ---- epilogue: fp8 scale, bias, one rounding, staged through LDS
  static_assert(NW * 32 * stage_pitch<CT, WTN>() <= S * STAGE, "epilogue staging");
  char *C = (char *)p.C + z * p.strideC * CE;
  store_tile_lds<CT, FM, FN>(acc, lds + wave * 32 * stage_pitch<CT, WTN>(), C, p.ldc, M, N, m0 + wm * WTM,
                             n0 + wn * WTN, p.bias, p.scale, lane);
}

template <int CT, bool NT>
hipError_t launch_quad8(const GemmParams &p, hipStream_t stream) {
  const int64_t tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
  hipLaunchKernelGGL((gemm_quad8_kernel<CT, NT>), dim3((unsigned)tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gemm_detail
}  // namespace tmm
