// Tiled GEMM on gfx950 matrix cores with four waves per 256x256 tile, each
// wave owning a 128x128 block of C (or 256x128 / 128x128 tiles of four
// waves): the kernel for 16-bit inputs, rows at any element alignment, whose
// K is a multiple of 64, at least 128 -- or, in its K-tail form (kQuadTail),
// any K with at least 128 below its last 64-element boundary, the last
// elements of K loaded and multiplied before the main loop.
//
//   C[z] = act(scale * A[z] . op(B[z]) (+ bias) (+ beta * old C[z])),
//   row-major, z < batch, act = identity or ReLU
//
// It keeps the four-stage LDS ring of gemm_ring.h (same stage size, same
// direct 16-byte global->LDS loads issued three K-steps ahead, same
// barrier-per-step protocol) and changes what runs on it, for two measured
// properties of the chip:
//   * LDS read bandwidth is the loop's limit with eight 128x64 waves: per
//     32-element K-step a CU reads 64 KiB of A fragments (each A row block
//     is read by the four waves sharing it) and 32 KiB of transposed B
//     fragments against 1024 matrix-core cycles per SIMD, at ~150 B/clk
//     (16-byte reads) and ~111 B/clk (transposing reads) per CU.  With four
//     waves of 128x128 each A block is read by two waves and each B block by
//     two: 32 KiB + 32 KiB, a third less.  That is the register blocking of
//     the Lecture 27 notes (section 2.4) taken to the largest block a wave
//     can hold: 256 fp32 accumulators per lane, kept in the accumulation
//     registers (AGPRs), with the fragments in the 256 architectural ones.
//   * Under random data the matrix cores run at the chip's power limit, and
//     the 16x16x32 instruction sustains a higher clock than the 32x32x16 one
//     for the same work (0.745 vs 0.68 of the dense peak in a register-only
//     loop on N(0,1) bf16 operands): it touches its accumulators once per 32
//     K instead of once per 16.  So each wave computes 8x8 blocks of 16x16.
// Fragments: lane l of a 16x16x32 block holds row (A) or column (B) l % 16
// and K elements 8 (l / 16) .. +7 of the step.
//   * A, and a K-contiguous B (trans_b): 16-byte reads of the stage's 64-byte
//     rows, chunk c of row r at c ^ qswz64(r) = c ^ ((r >> 1) & 3).  That
//     XOR was chosen by measurement: in a loop of such reads (lane l: row
//     l % 16, chunk l / 16) it shows no SQ_LDS_BANK_CONFLICT cycles and 188
//     B/clk per CU, against 50 % conflict cycles and 120 B/clk for
//     c ^ ((r >> 2) & 3) or no XOR.
//   * an N-contiguous B (NN): the stage holds k-rows of 256 elements as in
//     memory; the transposing read ds_read_b64_tr_b16 hands lane i of a
//     16-lane group the 4 elements (i mod 4) of the 8-byte pieces addressed
//     by lanes 4e + i / 4, so with lane s pointing at k-row k0 + s / 4,
//     columns n0 + 4 (s mod 4) .. +3, lane i receives B[k0 .. k0+3][n0 + i];
//     two such reads (k0 and k0 + 4) make a fragment.  The 32 lanes served
//     together read 8 k-rows (two groups of 4, 8 apart) x 32 bytes, so chunk
//     c of k-row r sits at c ^ (2 (r mod 4) + 8 ((r / 8) mod 2)): 16 distinct
//     positions among the 16 chunk slots of a 256-byte bank row.
// Within a step a wave issues its 64 matrix instructions row block by row
// block; after a row block's instructions it reads the next step's A
// fragment of that row block into the same registers, and between them the
// two halves of one of the next step's B fragments (into a second set, after
// the second and fifth instruction) and one of its eight direct loads (after
// the seventh), in an order fixed by scheduling fences.  (Other placements
// measured within 2 %; all eight loads in the first row block, 5-9 % slower.)
#pragma once

#include <type_traits>
#include <utility>

#include "gemm_mfma.h"
#include "gemm_ring.h"

namespace tmm {
namespace gemm_detail {

// s_waitcnt immediate waiting for vmcnt <= n only (lgkmcnt and expcnt at
// their maximum): a step's own LDS reads need not have landed at the
// barrier, only the direct loads that publish the next stage.
constexpr int vm_only_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// A (and NT B) stage: 16-byte chunk c of 64-byte row r at c ^ qswz64(r).
__device__ __forceinline__ int qswz64(int r) { return (r >> 1) & 3; }

// NN B stage for 16-wide fragments: 16-byte chunk c of k-row r at c ^ qswz(r).
__device__ __forceinline__ int qswz(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1); }

template <int AB>
__device__ __forceinline__ f32x4 mma16(const i32x4 &a, const i32x4 &b, const f32x4 &c) {
  if constexpr (AB == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Epilogue of a wave's (16 FM) x (16 FN) block held as FM x FN 16x16
// accumulators (lane l: column 16 j + l % 16, rows 16 i + 4 (l / 16) + r): in
// 32-row bands through the wave's LDS area `st` (rows quad_pitch bytes
// apart, 16 bytes of padding so the four 16-lane groups of a write land on
// distinct banks) as finished values (scale, bias, ReLU when RELU, one
// nearest-even rounding), then back 16 bytes per lane along the rows and out with
// whole-row stores, masked by M and N.
template <int CT, int FN>
constexpr int quad_pitch() { return 16 * FN * FmtBytes<CT>::value + 16; }

// 16 bytes to an address that is only element-aligned (rows of a C whose
// pitch is not a multiple of 16 bytes): one 16-byte store where it is 4-byte
// aligned, else a 2-byte store, three 4-byte stores and a 2-byte store, every
// access naturally aligned (a 2-byte store per element took 2 us more on the
// 4097 x 511 bf16 output).
typedef int i32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ void store16_elem_aligned(char *dst, const i32x4 &v) {
  if (((uintptr_t)dst & 3) == 0) {
    *(i32x4_a4 *)dst = v;
  } else {
    const uint32_t w0 = (uint32_t)v[0], w1 = (uint32_t)v[1], w2 = (uint32_t)v[2], w3 = (uint32_t)v[3];
    uint32_t *d = (uint32_t *)(dst + 2);
    *(uint16_t *)dst = (uint16_t)w0;
    d[0] = (w0 >> 16) | (w1 << 16);
    d[1] = (w1 >> 16) | (w2 << 16);
    d[2] = (w2 >> 16) | (w3 << 16);
    *(uint16_t *)(dst + 14) = (uint16_t)(w3 >> 16);
  }
}

template <int CT, int FM, int FN, bool RELU>
__device__ __forceinline__ void store_quad(const f32x4 (&acc)[FM][FN], char *st, char *C, int64_t ldc,
                                           int64_t M, int64_t N, int64_t row0, int64_t col0,
                                           const float *bias, float scale, int lane) {
  constexpr int CE = FmtBytes<CT>::value;
  constexpr int P = quad_pitch<CT, FN>();
  constexpr int CPR = 16 * FN * CE / 16;    // 16-byte pieces per row
  constexpr int EPC = 16 / CE;              // elements per piece
  constexpr int NRD = 32 * CPR / 64;        // read instructions per band
  static_assert(FM % 2 == 0 && NRD >= 1 && (32 * CPR) % 64 == 0, "epilogue geometry");
  const int c16 = lane & 15, g = lane >> 4;
  const bool vec = ((uintptr_t)C % 16) == 0 && ((ldc * CE) % 16) == 0;
  float bv[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = col0 + 16 * j + c16;
    bv[j] = (bias && col < N) ? bias[col] : 0.f;
  }
#pragma unroll
  for (int band = 0; band < FM / 2; ++band) {
    if (row0 + 32 * band >= M) break;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * ii + 4 * g + r;
          float v = acc[2 * band + ii][j][r] * scale + bv[j];
          if constexpr (RELU) v = v > 0.f ? v : 0.f;
          const uint32_t b = out_bits<CT>(v);
          char *d = st + row * P + (16 * j + c16) * CE;
          if constexpr (CE == 4) *(uint32_t *)d = b;
          else *(uint16_t *)d = (uint16_t)b;
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < NRD; ++t) {
      const int c = t * 64 + lane;
      const int row = c / CPR, pc = c % CPR;
      const i32x4 v = *(const i32x4 *)(st + row * P + pc * 16);
      const int64_t grow = row0 + 32 * band + row;
      const int64_t gcol = col0 + (int64_t)pc * EPC;
      if (grow >= M || gcol >= N) continue;
      char *dst = C + (grow * ldc + gcol) * CE;
      if (vec && gcol + EPC <= N) {
        __builtin_nontemporal_store(v, (i32x4 *)dst);
      } else if (gcol + EPC <= N) {
        store16_elem_aligned(dst, v);
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          if (gcol + e < N) {
            const uint32_t w = (uint32_t)v[(e * CE) / 4];
            if constexpr (CE == 4) ((uint32_t *)dst)[e] = w;
            else ((uint16_t *)dst)[e] = (uint16_t)(w >> (16 * (e & 1)));
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next band's writes
    __builtin_amdgcn_wave_barrier();
  }
}

// Full-form epilogue of the same block, C = act(alpha acc + bias + beta C_old),
// beta != 0: per 32-row band, the old C of the 4-column quads this lane will
// write is loaded first (as stored: 16-bit words or fp32, a vector load when
// C and its pitch allow), so that those loads are in flight while the fp32
// values (alpha acc + bias) are staged through LDS as above; then each quad
// is read back, beta C_old added, ReLU when act == 1, one nearest-even
// rounding, and stored.
template <int CT, int FN>
constexpr int quad_ex_pitch() { return 16 * FN * 4 + 16; }

template <int CT>
struct OldQuad { typedef uint64_t type; };  // four 16-bit words
template <>
struct OldQuad<kF32> { typedef f32x4 type; };

// Calls f(integral_constant<int, 0>), f(..1), ... in order while it
// returns true.
template <typename F, int... I>
__device__ __forceinline__ void for_each_index(F &f, std::integer_sequence<int, I...>) {
  (void)(... && f(std::integral_constant<int, I>()));
}

template <int CT, int FM, int FN>
__device__ __forceinline__ void store_quad_ex(const f32x4 (&acc)[FM][FN], char *st, char *C, int64_t ldc,
                                              int64_t M, int64_t N, int64_t row0, int64_t col0,
                                              const float *bias, float alpha, float beta, int act, int lane) {
  constexpr int CE = FmtBytes<CT>::value;
  constexpr int P = quad_ex_pitch<CT, FN>();
  constexpr int QPR = 4 * FN;               // 4-column quads per row
  constexpr int NRD = 32 * QPR / 64;        // quads per lane per band
  static_assert(FM % 2 == 0 && NRD >= 1, "epilogue geometry");
  typedef typename OldQuad<CT>::type Old;
  const int c16 = lane & 15, g = lane >> 4;
  const bool vec = ((uintptr_t)C % (4 * CE)) == 0 && (ldc % 4) == 0;
  float bv[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = col0 + 16 * j + c16;
    bv[j] = (bias && col < N) ? bias[col] : 0.f;
  }
  // one band per call, its index a constant: the accumulators are only ever
  // indexed by constants, so they stay in registers however large the body
  auto do_band = [&](auto band_c) -> bool {
    constexpr int band = decltype(band_c)::value;
    if (row0 + 32 * band >= M) return false;
    Old old[NRD];
#pragma unroll
    for (int t = 0; t < NRD; ++t) {
      const int qd = t * 64 + lane;
      const int64_t grow = row0 + 32 * band + qd / QPR;
      const int64_t gcol = col0 + (int64_t)(qd % QPR) * 4;
      const char *src = C + (grow * ldc + gcol) * CE;
      if (grow < M && gcol + 4 <= N && vec) {
        old[t] = *(const Old *)src;
      } else {
        Old w = {};
        if (grow < M) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (gcol + e < N) {
              if constexpr (CE == 4) w[e] = ((const float *)src)[e];
              else w |= (uint64_t)((const uint16_t *)src)[e] << (16 * e);
            }
          }
        }
        old[t] = w;
      }
    }
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *(float *)(st + (16 * ii + 4 * g + r) * P + (16 * j + c16) * 4) = acc[2 * band + ii][j][r] * alpha + bv[j];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < NRD; ++t) {
      const int qd = t * 64 + lane;
      const int lr = qd / QPR, qc = qd % QPR;
      f32x4 v = *(const f32x4 *)(st + lr * P + qc * 16);
      const int64_t grow = row0 + 32 * band + lr;
      const int64_t gcol = col0 + (int64_t)qc * 4;
      if (grow >= M || gcol >= N) continue;
      char *dst = C + (grow * ldc + gcol) * CE;
      f32x4 c;
      if constexpr (CE == 4) {
        c = old[t];
      } else {
        const uint64_t w = old[t];
        c = f32x4{in_value<CT>((uint16_t)w), in_value<CT>((uint16_t)(w >> 16)),
                  in_value<CT>((uint16_t)(w >> 32)), in_value<CT>((uint16_t)(w >> 48))};
      }
      v += beta * c;
      if (act == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = v[e] > 0.f ? v[e] : 0.f;
      }
      if (vec && gcol + 4 <= N) {
        if constexpr (CE == 4) {
          *(f32x4 *)dst = v;
        } else {
          const uint64_t w = (uint64_t)out_bits<CT>(v[0]) | ((uint64_t)out_bits<CT>(v[1]) << 16) |
                             ((uint64_t)out_bits<CT>(v[2]) << 32) | ((uint64_t)out_bits<CT>(v[3]) << 48);
          *(uint64_t *)dst = w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gcol + e < N) store_out<CT>(dst, e, v[e]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next band's writes
    __builtin_amdgcn_wave_barrier();
    return true;
  };
  for_each_index(do_band, std::make_integer_sequence<int, FM / 2>());
}

// Flag in EPI selecting the K-tail form (see the prologue): K need not be a
// multiple of 64, and an NN B's rows may end inside a 16-byte chunk.
constexpr int kQuadTail = 4;
// Flag in EPI selecting an eight-stage ring (128x128 tiles): seven steps in
// flight instead of three, for grids of one round of tiles, where each CU
// streams its own operand panels and the loads' latency, not the matrix
// work, sets the step time.
constexpr int kQuadDeep = 8;

// EPI, bits 0-1: 0 the plain epilogue, 1 the plain one with ReLU, 2 the
// full form (old C read back); bit 2: kQuadTail; bit 3: kQuadDeep.
template <int AB, int CT, bool NT, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_quad_kernel(GemmParams p) {
  constexpr bool TAIL = (EPI & kQuadTail) != 0;
  constexpr bool DEEP = (EPI & kQuadDeep) != 0;
  constexpr int EP = EPI & 3;
  constexpr int NW = 4;
  constexpr int WTM = BM / 2, WTN = BN / 2;     // each wave's block of C
  constexpr int FM = WTM / 16, FN = WTN / 16;   // 16x16 accumulators per wave
  constexpr int E = FmtBytes<AB>::value;
  constexpr int CE = FmtBytes<CT>::value;
  constexpr int ROWB = kRingRowBytes;           // 64 bytes of K per tile row per step
  constexpr int BK = ROWB / E;                  // 32
  constexpr int A_BYTES = BM * ROWB;
  constexpr int B_BYTES = BN * ROWB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int S = DEEP ? 8 : kRingStages;     // 4 (8)
  constexpr int NB_ROW = BN * E;                // NN: bytes of one k-row of the B stage
  constexpr int CPR = NB_ROW / 16, RPI = 64 / CPR;  // NN: chunks per k-row, k-rows per load
  constexpr int LA = A_BYTES / 1024 / NW;       // direct loads per wave per step (A)
  constexpr int LB = B_BYTES / 1024 / NW;       // (B)
  constexpr int LPS = LA + LB;
  static_assert(E == 2, "four-wave kernel: 16-bit inputs");
  static_assert((S == 4 || (S == 8 && BM == 128 && BN == 128)) && BK == 32, "geometry");
  static_assert((BM == 256 || BM == 128) && (BN == 256 || BN == 128) && FM >= FN, "tile shapes");
  static_assert(LPS <= FM, "one direct load per row block at most");
  // slots (instruction index within a row block) of the two B half-reads and the load
  constexpr int QB0 = 1, QB1 = FN >= 8 ? 4 : 3, QD = FN >= 8 ? 6 : 2;

  __shared__ __attribute__((aligned(16))) char lds[S * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  int64_t pid = remap_xcd(blockIdx.x, (int64_t)gridDim.x);
  const int64_t z = pid / tiles;
  pid -= z * tiles;
  int64_t tm, tn;
  group_order(pid, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const char *A = (const char *)p.A + z * p.strideA * E;
  const char *B = (const char *)p.B + z * p.strideB * E;

  // ---- direct-load sources (byte offsets < 4 GiB, checked by the host).
  // A and an NT B: instruction i of wave w fills stage rows w BM/4 + 16 i
  // ..+15; lane L lands at row L / 4, position L % 4 and loads logical chunk
  // (L % 4) ^ qswz64(row).  Rows past M (N) read the last valid row.
  uint32_t a_off[LA], b_off[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int row = wave * (BM / NW) + i * 16 + (lane >> 2);
    const int64_t r = min64(m0 + row, M - 1);
    a_off[i] = (uint32_t)(r * p.lda * E + (((lane & 3) ^ qswz64(row)) << 4));
  }
  if constexpr (NT) {
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = wave * (BN / NW) + i * 16 + (lane >> 2);
      const int64_t r = min64(n0 + row, N - 1);
      b_off[i] = (uint32_t)(r * p.ldb * E + (((lane & 3) ^ qswz64(row)) << 4));
    }
  } else {
    // NN: instruction i of wave w fills the RPI k-rows from 8 w + RPI i;
    // lane L lands at k-row L / CPR, position L % CPR and loads logical
    // chunk (L % CPR) ^ qswz(row).  A chunk wholly past N (the host ensures
    // N * E % 16 == 0) reads chunk 0 of the tile; it only feeds outputs that
    // are not stored.
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = wave * (BK / NW) + i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ qswz(row);
      const int64_t col = n0 + (int64_t)c * (16 / E);
      const int64_t ccol = col < N ? col : n0;
      b_off[i] = (uint32_t)(((int64_t)row * p.ldb + ccol) * E);
    }
  }
  const int64_t kstep_b = NT ? (int64_t)ROWB : (int64_t)BK * p.ldb * E;
  const uint32_t lds0 = lds_addr(lds);

  // ---- fragment addresses (bytes within a stage)
  const int l16 = lane & 15, G = lane >> 4;
  // A (and NT B): row block base + lane row l16, chunk G (swizzled)
  const int a_lane = l16 * ROWB + ((G ^ qswz64(l16)) << 4);
  const int a_base = wm * WTM * ROWB + a_lane;                   // + 1024 i
  const int bt_base = A_BYTES + wn * WTN * ROWB + a_lane;        // NT: + 1024 j
  // NN: lane (G, s = l16) reads k-row 8 G + 4 h + s / 4, columns
  // WTN wn + 16 j + 4 (s % 4) .. +3; see the header comment for the swizzle.
  // The wave's and the block's columns only flip bits of the 16 * qswz
  // field (or, for the wave of a 256-wide tile, a bit above it): address =
  // base ^ 2 WTN wn ^ 32 j.
  const int f = 2 * (l16 >> 2) + 8 * (G & 1);
  const int bn_base = (A_BYTES + (8 * G + (l16 >> 2)) * NB_ROW + 16 * ((l16 & 3) >> 1) + 8 * (l16 & 1) +
                       16 * f) ^ (2 * WTN * wn);

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  i32x4 fa[FM];
  i32x4 fb0[FN], fb1[FN];

  auto issue_one = [&](int64_t kt, int stage, int q) __attribute__((always_inline)) {
    const uint32_t la = lds0 + (uint32_t)(stage * STAGE);
    if (q < LA) {
      dma16(A + kt * ROWB + a_off[q], la + (wave * (BM / NW) + q * 16) * ROWB);
    } else {
      const int i = q - LA;
      if constexpr (NT)
        dma16(B + kt * kstep_b + b_off[i], la + A_BYTES + (wave * (BN / NW) + i * 16) * ROWB);
      else
        dma16(B + kt * kstep_b + b_off[i], la + A_BYTES + (wave * (BK / NW) + i * RPI) * NB_ROW);
    }
  };
  auto read_a = [&](int stage, int i) __attribute__((always_inline)) {
    fa[i] = *(const i32x4 *)(lds + stage * STAGE + a_base + i * 16 * ROWB);
  };
  // The next step's B fragment j, in two halves h = 0, 1 (NN: one
  // transposing read each; NT: one 16-byte read, at h = 0).
  i32x2 half_lo[FN];
  auto read_b = [&](int stage, i32x4 (&fb)[FN], int j, int h) __attribute__((always_inline)) {
    if constexpr (NT) {
      if (h == 0) fb[j] = *(const i32x4 *)(lds + stage * STAGE + bt_base + j * 16 * ROWB);
    } else {
      const char *pb = lds + stage * STAGE + (bn_base ^ (32 * j));
      if (h == 0) {
        half_lo[j] = __builtin_bit_cast(i32x2, lds_read_tr16(pb));
      } else {
        const i32x2 hi = __builtin_bit_cast(i32x2, lds_read_tr16(pb + 4 * NB_ROW));
        fb[j] = i32x4{half_lo[j][0], half_lo[j][1], hi[0], hi[1]};
      }
    }
  };

  // K-tail form: the last KT elements of K (K mod 64, or 64 when that is 0)
  // are not loaded by the ring; the host guarantees K - KT >= 4 BK.
  const int64_t KT = TAIL ? ((K & 63) ? (K & 63) : 64) : 0;
  const int64_t nsteps = (K - KT) / BK;  // the host guarantees an even count >= 4
  constexpr int D = S - 1;               // steps loaded ahead
  auto stage_of = [](int64_t k) { return (int)(k & (S - 1)); };
  const int64_t pro = min64(D, nsteps);
  if constexpr (TAIL) {
    // The tail -- two 32-element steps from k0 = K - KT, zero past K, and
    // for an NN B zero past N -- is read first, one 16-byte load per chunk
    // holding a valid element (load8_u16_tail: a chunk that K or N cuts is
    // loaded from where its last valid element ends it and shifted into
    // place, so no read leaves the operands: K - KT >= 128, and a cut NN row
    // holds N >= 8 elements).  Then the ring's first D steps go out as in
    // the plain form, and the tail passes one step at a time through the
    // last stage (which the ring's first step reloads), in the ring's
    // layout: a barrier publishes it, the waves multiply it, a second
    // barrier releases the stage.  The ring's loads stay below k-row
    // K - KT: whole chunks inside every row of A (and of a K-contiguous B),
    // and for an NN B the chunk a row's end cuts through reads at most 7
    // elements into the next k-row (which exists, and holds N >= 8
    // elements, checked by the host); those columns past N feed only
    // outputs that are never stored.  The tail's loads cost ~3.5 of the
    // 22 us of 4097 x 511 x 1023 NN bf16 (timing copies without them).
    const int64_t k0 = K - KT;
    constexpr int TQA = BM * 8 / 256;                      // tail chunks per thread (A)
    constexpr int TQB = NT ? BN * 8 / 256 : 64 * CPR / 256;  // (B)
    i32x4 ta[TQA], tb[TQB];
#pragma unroll
    for (int i = 0; i < TQA; ++i) {
      const int q = tid + 256 * i, rr = q >> 3, c8 = q & 7;
      const int64_t row = m0 + rr, k = k0 + 8 * c8;
      const int nv = row < M ? (int)max64(0, min64(8, K - k)) : 0;
      ta[i] = nv > 0 ? load8_u16_tail(A + (row * p.lda + k) * E, nv) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < TQB; ++i) {
      const int q = tid + 256 * i;
      if constexpr (NT) {
        const int rr = q >> 3, c8 = q & 7;
        const int64_t row = n0 + rr, k = k0 + 8 * c8;
        const int nv = row < N ? (int)max64(0, min64(8, K - k)) : 0;
        tb[i] = nv > 0 ? load8_u16_tail(B + (row * p.ldb + k) * E, nv) : i32x4{0, 0, 0, 0};
      } else {
        const int kr = q / CPR, c = q % CPR;
        const int64_t k = k0 + kr, col = n0 + 8 * c;
        const int nv = k < K ? (int)max64(0, min64(8, N - col)) : 0;
        tb[i] = nv > 0 ? load8_u16_tail(B + (k * p.ldb + col) * E, nv) : i32x4{0, 0, 0, 0};
      }
    }
    for (int64_t k = 0; k < pro; ++k)
#pragma unroll
      for (int q = 0; q < LPS; ++q) issue_one(k, (int)k, q);
    char *const ts = lds + (S - 1) * STAGE;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t == 1 && KT <= BK) break;
#pragma unroll
      for (int i = 0; i < TQA; ++i) {
        const int q = tid + 256 * i, rr = q >> 3, c8 = q & 7;
        if ((c8 >> 2) == t) *(i32x4 *)(ts + rr * ROWB + (((c8 & 3) ^ qswz64(rr)) << 4)) = ta[i];
      }
#pragma unroll
      for (int i = 0; i < TQB; ++i) {
        const int q = tid + 256 * i;
        if constexpr (NT) {
          const int rr = q >> 3, c8 = q & 7;
          if ((c8 >> 2) == t) *(i32x4 *)(ts + A_BYTES + rr * ROWB + (((c8 & 3) ^ qswz64(rr)) << 4)) = tb[i];
        } else {
          const int kr = q / CPR, c = q % CPR, r32 = kr & 31;
          if ((kr >> 5) == t) *(i32x4 *)(ts + A_BYTES + r32 * NB_ROW + ((c ^ qswz(r32)) << 4)) = tb[i];
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
      __syncthreads();
#pragma unroll
      for (int i = 0; i < FM; ++i) read_a(S - 1, i);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        read_b(S - 1, fb0, j, 0);
        read_b(S - 1, fb0, j, 1);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mma16<AB>(fa[i], fb0[j], acc[i][j]);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // every read of the stage done before it is rewritten
      __syncthreads();
    }
  } else {
    for (int64_t k = 0; k < pro; ++k)
#pragma unroll
      for (int q = 0; q < LPS; ++q) issue_one(k, (int)k, q);
  }
  // steps 0 and 1 landed (steps 2 .. D - 1 may still be in flight), then
  // published; the eight-stage ring always has nsteps >= 8
  if constexpr (DEEP) __builtin_amdgcn_s_waitcnt(vm_wait((D - 2) * LPS));
  else if (pro > 2) __builtin_amdgcn_s_waitcnt(vm_wait(LPS));
  else __builtin_amdgcn_s_waitcnt(vm_wait(0));
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) read_a(0, i);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    read_b(0, fb0, j, 0);
    read_b(0, fb0, j, 1);
  }

  // Step kt: matrix instructions from fa / cb; the next step's fragments into
  // fa (row block by row block, after its last use) and nb (fragment i in row
  // block i) -- on the last step a harmless read of a stale stage; with
  // LOAD, step kt + D's direct loads (load q in row block q) into the stage
  // step kt - 1 used.  Barrier b(kt) then publishes step kt + 2 (its loads
  // are waited for first -- WAIT of the loads issued later may stay in
  // flight).  No vector register depends on a branch: the loop runs the
  // steps that load, the last D are written out after it.
  auto step = [&](int64_t kt, const i32x4 (&cb)[FN], i32x4 (&nb)[FN], auto load_tag, auto wait_tag)
      __attribute__((always_inline)) {
    constexpr bool LOAD = decltype(load_tag)::value;
    constexpr int WAIT = decltype(wait_tag)::value;
    const int nxt = stage_of(kt + 1);
    const int lst = stage_of(kt + D);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[i][j] = mma16<AB>(fa[i], cb[j], acc[i][j]);
        if (i < FN && j == QB0) read_b(nxt, nb, i, 0);
        if (i < FN && j == QB1) read_b(nxt, nb, i, 1);
        if (LOAD && i < LPS && j == QD) issue_one(kt + D, lst, i);
        __builtin_amdgcn_sched_barrier(0);
      }
      read_a(nxt, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(vm_only_wait(WAIT));
    __builtin_amdgcn_s_barrier();
  };
  using Load = std::integral_constant<bool, true>;
  using NoLoad = std::integral_constant<bool, false>;
  // in flight after a loading step's barrier: steps kt + 3 .. kt + D
  using WaitLoad = std::integral_constant<int, (D - 2) * LPS>;
  // nsteps is even and >= D + 1 (the host sends other K elsewhere)
  int64_t kt = 0;
  for (; kt + D + 1 < nsteps; kt += 2) {
    step(kt, fb0, fb1, Load(), WaitLoad());
    step(kt + 1, fb1, fb0, Load(), WaitLoad());
  }
  step(kt, fb0, fb1, Load(), WaitLoad());
  // the last D steps: after step kt + 1 + r, steps up to kt + D remain
  auto last_steps = [&](auto r_c) __attribute__((always_inline)) {
    constexpr int r = decltype(r_c)::value;
    using Wait = std::integral_constant<int, (D - 3 - r > 0 ? D - 3 - r : 0) * LPS>;
    if constexpr (r % 2 == 0) step(kt + 1 + r, fb1, fb0, NoLoad(), Wait());
    else step(kt + 1 + r, fb0, fb1, NoLoad(), Wait());
    return true;
  };
  for_each_index(last_steps, std::make_integer_sequence<int, D>());

  // ---- epilogue (the loop's last barrier follows every LDS read of the stages)
  char *C = (char *)p.C + z * p.strideC * CE;
  if constexpr (EP == 2) {
    static_assert(NW * 32 * quad_ex_pitch<CT, FN>() <= S * STAGE, "epilogue staging");
    store_quad_ex<CT, FM, FN>(acc, lds + wave * 32 * quad_ex_pitch<CT, FN>(), C, p.ldc, M, N, m0 + wm * WTM,
                              n0 + wn * WTN, p.bias, p.scale, p.beta, p.act, lane);
  } else {
    static_assert(NW * 32 * quad_pitch<CT, FN>() <= S * STAGE, "epilogue staging");
    store_quad<CT, FM, FN, EP == 1>(acc, lds + wave * 32 * quad_pitch<CT, FN>(), C, p.ldc, M, N, m0 + wm * WTM,
                           n0 + wn * WTN, p.bias, p.scale, lane);
  }
}

template <int AB, int CT, bool NT, int BM, int BN, int TAIL>
hipError_t launch_quad(const GemmParams &p, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.batch;
  // each epilogue in its own instantiation, so the plain kernel's code is
  // what it was without the others; only beta != 0 reads the old C
  if (p.beta != 0.f)
    hipLaunchKernelGGL((gemm_quad_kernel<AB, CT, NT, BM, BN, 2 | TAIL>), dim3((unsigned)tiles), dim3(256), 0, stream, p);
  else if (p.act == 1)
    hipLaunchKernelGGL((gemm_quad_kernel<AB, CT, NT, BM, BN, 1 | TAIL>), dim3((unsigned)tiles), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_quad_kernel<AB, CT, NT, BM, BN, 0 | TAIL>), dim3((unsigned)tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// The eight-stage ring on 128x128 tiles (plain epilogue only).
template <int AB, int CT, bool NT, int TAIL>
hipError_t launch_quad_deep(const GemmParams &p, hipStream_t stream) {
  const int64_t tiles = ((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch;
  hipLaunchKernelGGL((gemm_quad_kernel<AB, CT, NT, 128, 128, TAIL | kQuadDeep>), dim3((unsigned)tiles), dim3(256),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace gemm_detail
}  // namespace tmm
