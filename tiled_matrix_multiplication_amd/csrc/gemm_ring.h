// Tiled GEMM on gfx950 matrix cores with a four-stage LDS ring: the main
// kernel for 256x256 output tiles when every operand row is 16-byte aligned
// and K is a multiple of the K-step.
//
//   C[z] = scale * A[z] . op(B[z]) (+ bias),  row-major, z < batch
//
// Against the two-stage kernel in gemm_mfma.h (which serves every other
// case), this one keeps global loads three K-steps ahead of their use:
//   * a K-step is 64 bytes of K per tile row (32 bf16/fp16, 64 fp8); a stage
//     holds A (256 rows x 64 B) and B (16 KiB), 32 KiB, and four stages fill
//     128 KiB of the 160 KiB LDS;
//   * both operands move global->LDS with 16-byte direct loads (no
//     registers): at step k each wave issues its share of step k+3 into the
//     stage step k-1 used, and before the step's barrier it waits only for
//     the loads of step k+2 (those of step k+3 stay in flight), so that the
//     fragments of step k+1 are read during step k -- the
//     pipelining the MLC GPU-programming tutorial (devtrends.cc review)
//     describes for TMA, and the double buffering of the Lecture 27 notes
//     section 2.5 taken one level deeper;
//   * A and a K-contiguous B (trans_b) keep 64-byte rows, chunk c of row r
//     at position c ^ ((r >> 2) & 3): 16 consecutive rows read at one chunk
//     fall on 16 distinct bank groups;
//   * an N-contiguous B (NN) is stored as it is in memory, k-rows of BN
//     elements, 16-byte chunk c of row r at c ^ nn_swz(r), and the MFMA's B
//     fragments (consecutive k of one column per lane) are read with the
//     gfx950 transposing LDS reads.  ds_read_b64_tr_b16: in a group of 16
//     lanes, output lane i, element e is element (i mod 4) of the 8 bytes
//     addressed by lane 4e + i/4, so pointing lane s at k-row k0 + s/4,
//     columns n0 + 4 (s mod 4) hands lane i B[k0 .. k0+3][n0 + i].
//     ds_read_b64_tr_b8: output lane i, byte e is byte (i mod 8) of lane
//     2e + i/8, so lane s at k-row k0 + s/2, columns n0 + 8 (s mod 2) hands
//     lane i B[k0 .. k0+7][n0 + i] (both layouts measured on gfx950);
//   * a step's fragments (both 16-byte k-slots of every A and B block) live
//     in one of two register sets; while the step's matrix instructions
//     run from one set, the next step's fragments are read into the other,
//     one or two reads after each instruction in an order fixed by
//     scheduling fences, the K loop unrolled twice to swap the sets
//     (16-bit: 16 instructions of 32x32x16 per step, slot-major; fp8: 8 of
//     32x32x64, each fed by both slots).  This measured 6-10 % faster than
//     interleaving with sched_group_barrier hints over one register set;
//   * NW = 8 waves (two per SIMD) each own a 128x64 block of C as 4x2
//     32x32 accumulators.  NW = 4 (one wave per SIMD, 128x128 blocks as
//     4x4: a third fewer LDS fragment reads per matrix instruction) also
//     compiles but measured much slower and is not dispatched.  Tile order
//     and edges as in gemm_mfma.h; the epilogue is store_tile_lds;
//   * TA: A stored K x M (the transposed operand of a weight gradient,
//     X^T . dY), 16-bit inputs.  Its stage is k-rows of BM elements placed
//     like the NN B stage, and its fragments come from the same transposing
//     reads (the instruction's A and B fragments share one lane layout), so
//     a transposed A costs LDS read rate, not a transposing copy.
#pragma once

#include "gemm_mfma.h"

namespace tmm {
namespace gemm_detail {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kRingStages = 4;
constexpr int kRingRowBytes = 64;  // bytes of K per tile row per step

__device__ __forceinline__ int swz64(int row) { return (row >> 2) & 3; }

// s_waitcnt immediate (gfx9 encoding): vmcnt(n) in bits 3:0 and 15:14,
// expcnt left at 7, lgkmcnt(0).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// 16-byte direct global->LDS load: lane L's 16 bytes land at LDS byte
// address m0 + 16 L.  Written as assembly so that the compiler does not
// track it: its own tracking of such loads makes every later transposing
// LDS read wait for all of them (vmcnt(0)), which would drain the ring.
// The kernel orders these loads itself (s_waitcnt before each barrier, and
// none left in flight at exit).  One wait state separates the M0 write from
// its use by an LDS DMA on gfx9.
__device__ __forceinline__ void dma16(const char *g, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(m0) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const char *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Transposing 8-byte LDS reads (see the header comment).  Kept out of
// lambdas for the same host-pass reason as load16_to_lds.
__device__ __forceinline__ s16x4 lds_read_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(__attribute__((address_space(3))) char *)p);
}
__device__ __forceinline__ i32x2 lds_read_tr8(const char *p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (lds_i32x2 *)(__attribute__((address_space(3))) char *)p);
}

// NN B stage: 16-byte chunk c of k-row r sits at position c ^ nn_swz(r).
// An 8-byte transposing read is served 32 lanes at a time (256 bytes, all
// 64 banks): 16-bit, 4 consecutive k-rows x 4 chunks; 8-bit, 8 consecutive
// k-rows x 2 adjacent chunks (an even one and the next).  The XOR puts
// those on 16 distinct chunk positions.  (For 8-bit, c ^ (r mod 8) mapped
// rows 2i and 2i+1 onto the same pair of positions: SQ_LDS_BANK_CONFLICT
// was 25 % of SQ_LDS_IDX_ACTIVE.)
template <int E>
__device__ __forceinline__ int nn_swz(int row) {
  return E == 2 ? 4 * (row & 3) : 2 * (row & 7);
}

template <int AB, int CT, bool NT, int NW, bool FULL, bool TA = false>
__global__ __launch_bounds__(64 * NW) void gemm_ring_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256;
  constexpr int E = FmtBytes<AB>::value;
  constexpr int CE = FmtBytes<CT>::value;
  constexpr int BK = kRingRowBytes / E;            // K per step
  constexpr int WGN = NW / 2, WTM = BM / 2, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;      // 4 x 2 accumulators per wave
  constexpr int A_BYTES = BM * kRingRowBytes;      // 16 KiB (TA: BK k-rows x BM*E B)
  constexpr int B_BYTES = BN * kRingRowBytes;      // 16 KiB (NT: BN rows x 64 B; NN: BK rows x BN*E B)
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int NB_ROW = BN * E;                   // NN: bytes of one k-row of the B stage
  constexpr int CPR = NB_ROW / 16, RPI = 64 / CPR; // NN: chunks per k-row, k-rows per load
  constexpr int NA_ROW = BM * E;                   // TA: bytes of one k-row of the A stage
  constexpr int CPR_A = NA_ROW / 16, RPI_A = 64 / CPR_A;
  constexpr int LA = A_BYTES / 1024 / NW;          // direct loads per wave per step (A)
  constexpr int LB = B_BYTES / 1024 / NW;          // (B)
  constexpr int LPS = LA + LB;
  static_assert(E == 2 || E == 1, "ring path: 16-bit and fp8 inputs (fp32 uses the two-stage kernel)");
  static_assert((NW == 8 || NW == 4) && LA == 16 / NW && LB == 16 / NW, "ring geometry");
  static_assert(!TA || E == 2, "transposed A: 16-bit inputs");

  __shared__ __attribute__((aligned(16))) char lds[kRingStages * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int g = lane >> 5, l32 = lane & 31;

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

  // ---- direct-load sources: byte offsets (< 4 GiB, checked by the host).
  // A (and NT B): instruction i of wave w fills stage rows w*32 + 16 i ..+15;
  // lane L lands at row L/4, position L%4 and loads logical chunk
  // (L%4) ^ swz64(row).
  uint32_t a_off[LA], b_off[LB];
  if constexpr (TA) {
    // A stored K x M: k-rows of NA_ROW bytes, placed like the NN B stage
    // (chunk c of k-row r at position c ^ nn_swz(r)); a chunk wholly past M
    // (the host ensures M*E % 16 == 0) reads chunk 0 of the tile instead.
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int row = wave * (BK / NW) + i * RPI_A + lane / CPR_A;
      const int c = (lane % CPR_A) ^ nn_swz<E>(row);
      const int64_t col = m0 + (int64_t)c * (16 / E);
      const int64_t ccol = col < M ? col : m0;
      a_off[i] = (uint32_t)(((int64_t)row * p.lda + ccol) * E);
    }
  } else {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int row = wave * (BM / NW) + i * 16 + (lane >> 2);
      const int64_t r = min64(m0 + row, M - 1);
      a_off[i] = (uint32_t)(r * p.lda * E + (((lane & 3) ^ swz64(row)) << 4));
    }
  }
  if constexpr (NT) {
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = wave * (BN / NW) + i * 16 + (lane >> 2);
      const int64_t r = min64(n0 + row, N - 1);
      b_off[i] = (uint32_t)(r * p.ldb * E + (((lane & 3) ^ swz64(row)) << 4));
    }
  } else {
    // NN: k-rows of NB_ROW bytes (CPR chunks); instruction i of wave w
    // fills the RPI k-rows from w*BK/NW + i*RPI; lane L lands at row L/CPR,
    // position L%CPR and loads logical chunk (L%CPR) ^ nn_swz(row).  A chunk
    // wholly past N (the host ensures N*E % 16 == 0) reads chunk 0 instead;
    // it only feeds outputs that are never stored.
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = wave * (BK / NW) + i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ nn_swz<E>(row);
      const int64_t col = n0 + (int64_t)c * (16 / E);
      const int64_t ccol = col < N ? col : n0;
      b_off[i] = (uint32_t)(((int64_t)row * p.ldb + ccol) * E);
    }
  }
  const int64_t kstep_b = NT ? (int64_t)kRingRowBytes : (int64_t)BK * p.ldb * E;
  const int64_t kstep_a = TA ? (int64_t)BK * p.lda * E : (int64_t)kRingRowBytes;

  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int64_t kt, int stage) __attribute__((always_inline)) {
    const uint32_t la = lds0 + (uint32_t)(stage * STAGE);
    const char *ak = A + kt * kstep_a;
    const char *bk = B + kt * kstep_b;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      if constexpr (TA)
        dma16(ak + a_off[i], la + (wave * (BK / NW) + i * RPI_A) * NA_ROW);
      else
        dma16(ak + a_off[i], la + (wave * (BM / NW) + i * 16) * kRingRowBytes);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      if constexpr (NT)
        dma16(bk + b_off[i], la + A_BYTES + (wave * (BN / NW) + i * 16) * kRingRowBytes);
      else
        dma16(bk + b_off[i], la + A_BYTES + (wave * (BK / NW) + i * RPI) * NB_ROW);
    }
  };

  // ---- fragment reads.  k-slot s (0, 1) of a step: lane group g reads chunk
  // 2s + g of its A row (8 elements of K).
  // Block bases are multiples of 32 rows, so swz64(base + l32) = swz64(l32).
  const int a_frag = (wm * WTM + l32) * kRingRowBytes;
  int a_ch[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) a_ch[s] = ((2 * s + g) ^ swz64(l32)) << 4;
  // NN transposing reads: lane (G = lane/16, q = lane%16) of a 32-column block
  // starting at column jb reads k-row 16 s + 8 (G/2) + 4 h + q/4, columns
  // jb + 16 (G%2) + 4 (q%4) .. +3 (h = 0, 1 gives 8 consecutive k).
  const int G = lane >> 4, q = lane & 15;
  const int tr_row0 = 8 * (G >> 1) + (q >> 2);       // + 16 s + 4 h
  const int tr_col0 = wn * WTN + 16 * (G & 1) + 4 * (q & 3);  // + 32 j (elements)
  const int tr_acol0 = wm * WTM + 16 * (G & 1) + 4 * (q & 3); // TA: + 32 i

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Fenced ping-pong schedule: the fragments of a whole step live in one
  // of two register sets, (ca, cb)
  // for this step and (na, nb) for the next, swapped by unrolling the K loop
  // twice.  fp8: one 32x32x64 instruction per block fed by both k-slots
  // (chunks g and 2 + g of the 64-byte row: the same k order for A and B);
  // 16-bit: one 32x32x16 instruction per block and k-slot.
  typedef i32x4 FragA[2][FM];
  typedef i32x4 FragB[2][FN];
  constexpr int NMS = (E == 1 ? 1 : 2) * FM * FN;  // matrix instructions per step
  auto mma_u = [&](const FragA &ca, const FragB &cb, int u) __attribute__((always_inline)) {
    if constexpr (E == 1) {
      const int i = u / FN, j = u % FN;
      const i32x4 a0 = ca[0][i], a1 = ca[1][i], b0 = cb[0][j], b1 = cb[1][j];
      const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const i32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      // format code 0 (fp8 E4M3) for both operands; zero scale operands
      // select the unscaled instruction
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, 0, 0, 0, 0);
    } else {
      const int s2 = u / (FM * FN), i = (u % (FM * FN)) / FN, j = u % FN;
      if constexpr (AB == kBF16)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ca[s2][i]),
                                                            __builtin_bit_cast(bf16x8, cb[s2][j]),
                                                            acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ca[s2][i]),
                                                           __builtin_bit_cast(f16x8, cb[s2][j]),
                                                           acc[i][j], 0, 0, 0);
    }
  };
  // Read number r (0 .. NRS-1) of a step's fragments: first B, then A (one
  // 16-byte read per slot and block).  B, NT: one 16-byte read per slot.
  // B, NN, fp8: four 8-bit transposing reads per block, piece t holding
  // k 32 (t/2) + 16 g + 8 (t%2) .. +7 of the lane's column (lane (G, q) of a
  // 16-lane group points at k-row (piece base) + q/2, columns (block) +
  // 16 (G%2) + 8 (q%2) .. +7).  B, NN, 16-bit: four 16-bit transposing
  // reads per block, piece t = 2 s + h holding k 16 s + 8 g + 4 h .. +3.
  // A, TA: the same four transposing reads per block as B, NN, since the
  // instruction's A and B fragments have one layout (lane l: row / column
  // l % 32, k 8 (l / 32) .. +7).
  constexpr int RBS = FN * (NT ? 2 : 4);
  constexpr int NRS = RBS + (TA ? 4 : 2) * FM;
  i32x2 pcs[FN][4];
  i32x2 pca[FM][4];
  auto read_r = [&](int stage, FragA &na, FragB &nb, int r) __attribute__((always_inline)) {
    const char *base = lds + stage * STAGE;
    if (r >= RBS) {
      if constexpr (TA) {
        const int i = (r - RBS) >> 2, t = (r - RBS) & 3;
        const int row = 16 * (t >> 1) + 4 * (t & 1) + tr_row0;
        const int col = tr_acol0 + 32 * i;
        const int chunk = (col * E) >> 4, within = (col * E) & 15;
        pca[i][t] = __builtin_bit_cast(
            i32x2, lds_read_tr16(base + row * NA_ROW + ((chunk ^ nn_swz<E>(row)) << 4) + within));
        if (t & 1) {
          const int s2 = t >> 1;
          na[s2][i] = i32x4{pca[i][t - 1][0], pca[i][t - 1][1], pca[i][t][0], pca[i][t][1]};
        }
      } else {
        const int i = (r - RBS) >> 1, s2 = (r - RBS) & 1;
        na[s2][i] = *(const i32x4 *)(base + a_frag + i * 32 * kRingRowBytes + a_ch[s2]);
      }
    } else if constexpr (NT) {
      const int j = r >> 1, s2 = r & 1;
      nb[s2][j] = *(const i32x4 *)(base + A_BYTES + (wn * WTN + j * 32 + l32) * kRingRowBytes + a_ch[s2]);
    } else {
      const int j = r >> 2, t = r & 3;
      if constexpr (E == 1) {
        const int row = 32 * (t >> 1) + 16 * g + 8 * (t & 1) + (q >> 1);
        const int chunk = (wn * WTN + j * 32) / 16 + (G & 1);
        pcs[j][t] = lds_read_tr8(base + A_BYTES + row * NB_ROW + ((chunk ^ nn_swz<E>(row)) << 4) + 8 * (q & 1));
        if (t == 3) {
          nb[0][j] = i32x4{pcs[j][0][0], pcs[j][0][1], pcs[j][1][0], pcs[j][1][1]};
          nb[1][j] = i32x4{pcs[j][2][0], pcs[j][2][1], pcs[j][3][0], pcs[j][3][1]};
        }
      } else {
        const int row = 16 * (t >> 1) + 4 * (t & 1) + tr_row0;
        const int col = tr_col0 + 32 * j;
        const int chunk = (col * E) >> 4, within = (col * E) & 15;
        pcs[j][t] = __builtin_bit_cast(
            i32x2, lds_read_tr16(base + A_BYTES + row * NB_ROW + ((chunk ^ nn_swz<E>(row)) << 4) + within));
        if (t & 1) {
          const int s2 = t >> 1;
          nb[s2][j] = i32x4{pcs[j][t - 1][0], pcs[j][t - 1][1], pcs[j][t][0], pcs[j][t][1]};
        }
      }
    }
  };
  FragA fa0, fa1;
  FragB fb0, fb1;

  // waits that leave at most two, one or no step's loads in flight
  constexpr int kWait2 = vm_wait(2 * LPS);
  constexpr int kWait1 = vm_wait(LPS);
  constexpr int kWait0 = vm_wait(0);
  static_assert(2 * LPS < 64, "vmcnt field");

  // Wait for step `next`'s loads when the newest issued step is `newest`
  // (at most D - 2 steps later).
  auto wait_for = [&](int64_t next, int64_t newest) __attribute__((always_inline)) {
    if (kRingStages > 4 && newest > next + 1) __builtin_amdgcn_s_waitcnt(kWait2);
    else if (newest > next) __builtin_amdgcn_s_waitcnt(kWait1);
    else __builtin_amdgcn_s_waitcnt(kWait0);
  };
  constexpr int D = kRingStages - 1;  // steps loaded ahead
  auto stage_of = [](int64_t k) { return (int)(k % kRingStages); };

  const int64_t nsteps = K / BK;  // the host guarantees K % BK == 0, K > 0
  // Barrier b(k), at the end of step k, publishes step k+2: the fragments of
  // step k+1 can then be read during step k, under its matrix instructions,
  // and no LDS read waits behind a barrier.  Stage (k+D) mod S, which step k
  // loads, was last read during step k-1, before b(k-1).
  const int64_t pro = min64(kRingStages - 1, nsteps);
  for (int64_t k = 0; k < pro; ++k) issue(k, (int)k);
  wait_for(1, pro - 1);
  __syncthreads();
  {
    // Step kt reads step kt+1's fragments (on the last step a harmless read
    // of a stale stage) into the other register set, RPM reads after each of
    // the first three quarters of the matrix instructions (so the reads have
    // landed when the barrier's lgkmcnt(0) comes), in the order written
    // (scheduling fences).
    constexpr int RW = NMS - NMS / 4;
    constexpr int RPM = (NRS + RW - 1) / RW;
#pragma unroll
    for (int r = 0; r < NRS; ++r) read_r(0, fa0, fb0, r);
    auto step_f = [&](int64_t kt, const FragA &ca, const FragB &cb, FragA &na, FragB &nb)
        __attribute__((always_inline)) {
      if (kt + D < nsteps) issue(kt + D, stage_of(kt + D));
      const int nxt = stage_of(kt + 1);
#pragma unroll
      for (int u = 0; u < NMS; ++u) {
        mma_u(ca, cb, u);
#pragma unroll
        for (int r = u * RPM; r < (u + 1) * RPM && r < NRS; ++r) read_r(nxt, na, nb, r);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_for(kt + 2, min64(kt + D, nsteps - 1));
      __syncthreads();
    };
    for (int64_t kt = 0; kt < nsteps; kt += 2) {
      step_f(kt, fa0, fb0, fa1, fb1);
      if (kt + 1 < nsteps) step_f(kt + 1, fa1, fb1, fa0, fb0);
    }
  }

  // ---- epilogue: fp8 scale, bias, round once, masked store (staged through LDS)
  char *C = (char *)p.C + z * p.strideC * CE;
  // the loop's last barrier follows every LDS read of the stages
  static_assert(NW * 32 * stage_pitch<CT, WTN>() <= kRingStages * STAGE, "epilogue staging");
  if constexpr (FULL) {
    static_assert(NW * 16 * (WTN * 4 + 32) <= kRingStages * STAGE, "full-form epilogue staging");
    store_tile_ex<CT, FM, FN>(acc, lds + wave * 16 * (WTN * 4 + 32), C, p.ldc, M, N, m0 + wm * WTM,
                              n0 + wn * WTN, p.bias, p.scale, p.beta, p.act, lane);
  } else {
    store_tile_lds<CT, FM, FN>(acc, lds + wave * 32 * stage_pitch<CT, WTN>(), C, p.ldc, M, N,
                               m0 + wm * WTM, n0 + wn * WTN, p.bias, p.scale, lane);
  }
}

// A stored K x M (16-bit inputs); the host ensures M*E % 16 == 0, 16-byte
// aligned rows of A and B and K % 32 == 0.
template <int AB, int CT, bool NT>
hipError_t launch_ring_ta(const GemmParams &p, hipStream_t stream) {
  const int64_t tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
  if (p.beta != 0.f || p.act != 0)
    hipLaunchKernelGGL((gemm_ring_kernel<AB, CT, NT, 8, true, true>), dim3((unsigned)tiles), dim3(512), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((gemm_ring_kernel<AB, CT, NT, 8, false, true>), dim3((unsigned)tiles), dim3(512), 0,
                       stream, p);
  return hipGetLastError();
}

template <int AB, int CT, bool NT, int NW>
hipError_t launch_ring(const GemmParams &p, hipStream_t stream) {
  const int64_t tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
  if (p.beta != 0.f || p.act != 0)
    hipLaunchKernelGGL((gemm_ring_kernel<AB, CT, NT, NW, true>), dim3((unsigned)tiles), dim3(64 * NW), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((gemm_ring_kernel<AB, CT, NT, NW, false>), dim3((unsigned)tiles), dim3(64 * NW), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace gemm_detail
}  // namespace tmm
