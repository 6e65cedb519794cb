// Tiled GEMM on gfx950 matrix cores (MFMA), fp32 accumulation: the kernel
// template.  Each gemm_<type>.hip instantiates it for one input type.
//
//   C[z] = scale * A[z] . op(B[z]) (+ bias),  row-major, z < batch
//
// Structure (each piece is the gfx950 form of a step the pages describe):
//   * C is cut into BM x BN tiles, one 256-lane workgroup (4 waves of 64) per
//     tile; each K-step moves a BM x BK slice of A and a BK x BN slice of
//     op(B) into LDS and reuses it BN resp. BM times ("GEMM to FlashAttention"
//     page, tiling figure and tiled_matmul listing; devpress GPU notes
//     section 3.6, tiling cuts global reads by the tile width).
//   * Global loads are 16 bytes per lane with neighbouring lanes on
//     neighbouring addresses (devpress notes section 3.5, coalescing).
//   * LDS rows are 128 bytes (one K-step of any element type: 64 bf16/fp16,
//     128 fp8, 32 fp32) made of eight 16-byte chunks; chunk c of row r is
//     stored at chunk position c ^ swz(r), so the 16-byte fragment reads of
//     consecutive rows and the transposing writes hit distinct banks (the
//     swizzle-against-bank-conflicts idea of the MLC GPU-programming
//     tutorial reviewed on devtrends.cc).
//   * Two LDS stages: the global loads of K-step k+1 are issued before the
//     matrix instructions of step k and written to the other stage after
//     them, one barrier per step (Lecture 27 notes section 2.5: double
//     buffering trades on-chip space for overlap).
//   * Each wave owns a (BM/2) x (BN/2) block of C as a grid of 32x32 MFMA
//     accumulators in registers (register blocking, Lecture 27 notes
//     section 2.4; matrix instructions instead of scalar FMAs, section 2.8;
//     low-precision inputs with fp32 accumulation, section 2.7).
//   * Epilogue: fp8 dequantisation scale, bias per output column, one
//     round-to-nearest-even conversion, masked stores (the fused epilogue of
//     the Lecture 27 fused-convolution listing; bias per output feature from
//     the linear-layer formula of the GEMM page).  A store instruction
//     writes two rows x 32 columns: whole 128-byte lines for fp32 output.
//   * Edges: rows past M (columns past N) of A (op(B)) are read from the
//     last valid row, which only feeds outputs that are never stored; the K
//     tail is zero-filled; stores are masked (tiled_matmul's min() bounds).
//   * Tile order: workgroups are spread round-robin over the 8 XCDs, so the
//     tile index is remapped to give each XCD a contiguous run of tiles,
//     grouped 4 tile-rows deep so the run shares A and B panels in that
//     XCD's L2 (devpress notes section 3.7 on tiles versus compute units).
#pragma once

#include "load_words.h"
#include "tmm_internal.h"

namespace tmm {
namespace gemm_detail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int F> struct FmtBytes;
template <> struct FmtBytes<kF32> { static constexpr int value = 4; };
template <> struct FmtBytes<kBF16> { static constexpr int value = 2; };
template <> struct FmtBytes<kF16> { static constexpr int value = 2; };
template <> struct FmtBytes<kF8> { static constexpr int value = 1; };

constexpr int kRowBytes = 128;  // bytes of one K-step per tile row
constexpr int kGroupM = 4;      // tile-rows per ordering group

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

// Chunk swizzle of LDS row `row`: logical chunk c is stored at position
// c ^ swz(row).  Any 8 consecutive rows, and any 8 rows spaced 8 apart, get 8
// distinct values, so 16-byte fragment reads of consecutive rows and the NN
// transpose writes (rows 8 apart per lane) spread over all banks.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

// load8_u16_words: the misaligned 16-bit piece loader of load_words.h.

// Elements [0, nvalid) of the 16-byte chunk at p (element-aligned); zero past them.
template <int E>
__device__ __forceinline__ i32x4 load_chunk_elems(const char *p, int nvalid) {
  if constexpr (E == 2) return load8_u16_words(p, nvalid);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 16 / E; ++e) {
    if (e < nvalid) {
      uint32_t v;
      if constexpr (E == 1)
        v = *(const uint8_t *)(p + e);
      else if constexpr (E == 2)
        v = *(const uint16_t *)(p + 2 * e);
      else
        v = *(const uint32_t *)(p + 4 * e);
      w[(e * E) >> 2] |= v << (8 * ((e * E) & 3));
    }
  }
  return i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

__device__ __forceinline__ i32x4 load16(const char *p) { return *(const i32x4 *)p; }

// 16 bytes per lane from global memory straight into LDS: lane L of the wave
// writes lds_wave_base + 16 L (gfx950 global_load_lds_dwordx4).  Kept out of
// lambdas: inside one, hipcc's host pass drops the kernel's launch stub.
__device__ __forceinline__ void load16_to_lds(const char *g, char *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, lds_wave_base, 16, 0, 0);
}

// Workgroups go to XCD (id mod 8).  Give XCD x the contiguous tile run
// [x*n/8, (x+1)*n/8) for the part of the grid that fills whole rounds.
__device__ __forceinline__ int64_t remap_xcd(int64_t pid, int64_t n) {
  const int64_t per = n >> 3;
  if (pid >= (per << 3)) return pid;
  return (pid & 7) * per + (pid >> 3);
}

// Tile t of a tm_count x tn_count grid, visited kGroupM tile-rows at a time.
__device__ __forceinline__ void group_order(int64_t t, int64_t tm_count, int64_t tn_count,
                                            int64_t &tm, int64_t &tn) {
  const int64_t per_group = (int64_t)kGroupM * tn_count;
  const int64_t group = t / per_group;
  const int64_t first = group * kGroupM;
  const int64_t rows = min64((int64_t)kGroupM, tm_count - first);
  const int64_t in = t - group * per_group;
  tm = first + in % rows;
  tn = in / rows;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: nearest-even, subnormals kept
  return __builtin_bit_cast(uint16_t, h);
}

template <int CT>
__device__ __forceinline__ void store_out(char *C, int64_t idx, float v) {
  if constexpr (CT == kF32)
    ((float *)C)[idx] = v;
  else if constexpr (CT == kBF16)
    ((uint16_t *)C)[idx] = f32_to_bf16_rne(v);
  else
    ((uint16_t *)C)[idx] = f32_to_f16_rne(v);
}

// Value of a stored 16-bit output element (the old C of the full form).
template <int CT>
__device__ __forceinline__ float in_value(uint16_t u) {
  if constexpr (CT == kBF16) return __uint_as_float((uint32_t)u << 16);
  else return (float)__builtin_bit_cast(_Float16, u);
}

// Output bits of v in the output type (fp32, or bf16 / fp16 nearest-even).
template <int CT>
__device__ __forceinline__ uint32_t out_bits(float v) {
  if constexpr (CT == kF32) return __float_as_uint(v);
  else if constexpr (CT == kBF16) return f32_to_bf16_rne(v);
  else return f32_to_f16_rne(v);
}

// Row pitch (bytes) of a wave's epilogue staging area for WT columns.
// fp32: the row plus 32 bytes, so rows r and r + 4 (one store instruction
// of the accumulator layout) start 32 banks apart.  16-bit rows of 8 or more
// 16-byte pieces: no padding, and piece p of row r sits at p ^ stage_swz(r)
// instead -- rows r and r + 4 (one write instruction) put their 4 pieces
// in disjoint halves of the row, and each 16 lanes of a read-back take 256
// contiguous bytes (two 128-byte rows or one 256-byte row).  The padded
// 16-bit pitch left two rows of one read on the same banks:
// SQ_LDS_BANK_CONFLICT was 20-25 % of SQ_LDS_IDX_ACTIVE where this
// epilogue weighs (batched 2048 x 2048 x 128 fp16 out).
template <int CT, int WT>
constexpr bool stage_swizzled() { return FmtBytes<CT>::value == 2 && WT * 2 / 16 >= 8; }
template <int CT, int WT>
constexpr int stage_pitch() {
  return stage_swizzled<CT, WT>() ? WT * 2 : WT * FmtBytes<CT>::value + 32;
}
template <int CT, int WT>
__device__ __forceinline__ int stage_swz(int row) {
  return stage_swizzled<CT, WT>() ? 4 * ((row >> 2) & 1) : 0;
}

// Epilogue through LDS.  For each 32-row band i of the wave's block, the
// accumulators go to the wave's own LDS area `st` (32 rows, stage_pitch
// bytes apart) as finished output values (v = scale * acc + bias, rounded
// once), then come back 16 bytes per lane along the rows, so every global
// store instruction writes whole row segments (4 rows of 256 bytes for a
// 64-column fp32 block) instead of 32-column pieces of two rows.  Stores are
// masked by M and N; a 16-byte piece that crosses N, or any piece when C or
// its row pitch is not 16-byte aligned, is stored element by element.  The
// caller has finished every LDS read of the main loop (barrier) before this.
template <int CT, int FM, int FN>
__device__ __forceinline__ void store_tile_lds(const f32x16 (&acc)[FM][FN], char *st, char *C,
                                               int64_t ldc, int64_t M, int64_t N, int64_t row0,
                                               int64_t col0, const float *bias, float scale,
                                               int lane) {
  constexpr int CE = FmtBytes<CT>::value;
  constexpr int WT = FN * 32;                 // columns of the wave's block
  constexpr int RB = WT * CE;                 // bytes of one row of it
  constexpr int P = stage_pitch<CT, WT>();
  constexpr int CPR = RB / 16;                // 16-byte pieces per row
  constexpr int EPC = 16 / CE;                // elements per piece
  constexpr int NRD = 32 * CPR / 64;          // read instructions per band
  static_assert(NRD >= 1 && (32 * CPR) % 64 == 0, "epilogue geometry");
  const int l32 = lane & 31, g = lane >> 5;
  const bool vec = ((uintptr_t)C % 16) == 0 && ((ldc * CE) % 16) == 0;
  float bv[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = col0 + j * 32 + l32;
    bv[j] = (bias && col < N) ? bias[col] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (row0 + i * 32 >= M) break;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * g + (r & 3);
        const uint32_t b = out_bits<CT>(acc[i][j][r] * scale + bv[j]);
        const int byte = (j * 32 + l32) * CE;
        char *d = st + row * P + ((((byte >> 4) ^ stage_swz<CT, WT>(row)) << 4) | (byte & 15));
        if constexpr (CE == 4) *(uint32_t *)d = b;
        else *(uint16_t *)d = (uint16_t)b;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < NRD; ++t) {
      const int c = t * 64 + lane;
      const int row = c / CPR, pc = c % CPR;
      const i32x4 v = *(const i32x4 *)(st + row * P + ((pc ^ stage_swz<CT, WT>(row)) << 4));
      const int64_t grow = row0 + i * 32 + row;
      const int64_t gcol = col0 + (int64_t)pc * EPC;
      if (grow >= M || gcol >= N) continue;
      char *dst = C + (grow * ldc + gcol) * CE;
      if (vec && gcol + EPC <= N) {
        // non-temporal: C is written once and not read back here
        __builtin_nontemporal_store(v, (i32x4 *)dst);
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

// Full-form epilogue, C = act(alpha * acc + bias + beta * C_old): the
// same staging through the wave's LDS area, but as fp32 values and in
// 16-row halves of each 32-row band (so the area is 16 rows of WT * 4 + 32
// bytes), then back 4 columns per lane: the old C of those 4 columns is
// read when beta != 0, added, ReLU applied when act == 1, one
// nearest-even rounding, and the 4 outputs stored.  Vector loads and
// stores need C and its row pitch aligned to 4 elements.
template <int CT, int FM, int FN>
__device__ __forceinline__ void store_tile_ex(const f32x16 (&acc)[FM][FN], char *st, char *C,
                                              int64_t ldc, int64_t M, int64_t N, int64_t row0,
                                              int64_t col0, const float *bias, float alpha,
                                              float beta, int act, int lane) {
  constexpr int CE = FmtBytes<CT>::value;
  constexpr int WT = FN * 32;                 // columns of the wave's block
  constexpr int P = WT * 4 + 32;              // fp32 staging row pitch (bytes)
  constexpr int QPR = WT / 4;                 // 4-column quads per row
  constexpr int NRD = 16 * QPR / 64;          // read instructions per 16-row half
  static_assert(NRD >= 1 && (16 * QPR) % 64 == 0, "epilogue geometry");
  const int l32 = lane & 31, g = lane >> 5;
  const bool vec = ((uintptr_t)C % (4 * CE)) == 0 && (ldc % 4) == 0;
  float bv[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = col0 + j * 32 + l32;
    bv[j] = (bias && col < N) ? bias[col] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (row0 + i * 32 + hh * 16 >= M) break;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int r = 8 * hh; r < 8 * hh + 8; ++r) {
          const int lr = 8 * ((r >> 2) & 1) + 4 * g + (r & 3);   // row within the half
          *(float *)(st + lr * P + (j * 32 + l32) * 4) = acc[i][j][r] * alpha + bv[j];
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int t = 0; t < NRD; ++t) {
        const int q = t * 64 + lane;
        const int lr = q / QPR, qc = q % QPR;
        f32x4 v = *(const f32x4 *)(st + lr * P + qc * 16);
        const int64_t grow = row0 + i * 32 + hh * 16 + lr;
        const int64_t gcol = col0 + (int64_t)qc * 4;
        if (grow >= M || gcol >= N) continue;
        char *dst = C + (grow * ldc + gcol) * CE;
        const bool full = vec && gcol + 4 <= N;
        if (beta != 0.f) {
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
          if (full) {
            if constexpr (CE == 4) {
              c = *(const f32x4 *)dst;
            } else {
              const uint64_t w = *(const uint64_t *)dst;
              c = f32x4{in_value<CT>((uint16_t)w), in_value<CT>((uint16_t)(w >> 16)),
                        in_value<CT>((uint16_t)(w >> 32)), in_value<CT>((uint16_t)(w >> 48))};
            }
          } else {
            if constexpr (CE == 4) {
              if (gcol + 0 < N) c[0] = ((const float *)dst)[0];
              if (gcol + 1 < N) c[1] = ((const float *)dst)[1];
              if (gcol + 2 < N) c[2] = ((const float *)dst)[2];
              if (gcol + 3 < N) c[3] = ((const float *)dst)[3];
            } else {
              if (gcol + 0 < N) c[0] = in_value<CT>(((const uint16_t *)dst)[0]);
              if (gcol + 1 < N) c[1] = in_value<CT>(((const uint16_t *)dst)[1]);
              if (gcol + 2 < N) c[2] = in_value<CT>(((const uint16_t *)dst)[2]);
              if (gcol + 3 < N) c[3] = in_value<CT>(((const uint16_t *)dst)[3]);
            }
          }
          v += beta * c;
        }
        if (act == 1) {
          v[0] = v[0] > 0.f ? v[0] : 0.f;
          v[1] = v[1] > 0.f ? v[1] : 0.f;
          v[2] = v[2] > 0.f ? v[2] : 0.f;
          v[3] = v[3] > 0.f ? v[3] : 0.f;
        }
        if (full) {
          if constexpr (CE == 4) {
            *(f32x4 *)dst = v;
          } else {
            const uint64_t w = (uint64_t)out_bits<CT>(v[0]) | ((uint64_t)out_bits<CT>(v[1]) << 16) |
                               ((uint64_t)out_bits<CT>(v[2]) << 32) |
                               ((uint64_t)out_bits<CT>(v[3]) << 48);
            *(uint64_t *)dst = w;
          }
        } else {
          if (gcol + 0 < N) store_out<CT>(dst, 0, v[0]);
          if (gcol + 1 < N) store_out<CT>(dst, 1, v[1]);
          if (gcol + 2 < N) store_out<CT>(dst, 2, v[2]);
          if (gcol + 3 < N) store_out<CT>(dst, 3, v[3]);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next half's writes
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Matrix instructions of one K-step (128 bytes of K per row), numbered
// 0 .. units<AB>(FM, FN) - 1 in issue order.  fa[s][i] / fb[s][j] hold, for
// k-slot s = 0..3, the 16-byte chunk 2s + (lane / 32) of the lane's A row /
// B column; A and B use the same slot-to-chunk map, so each instruction
// pairs equal k indices.
//   bf16 / fp16: 32x32x16, one slot per instruction, unit = (s, i, j)
//   fp8 e4m3:    32x32x64, 32 bytes of K per lane = slots 2h and 2h+1,
//                unit = (h, i, j)
//   fp32:        32x32x2, one float per lane, a slot holds 4 floats,
//                unit = (s, t, i, j)
template <int AB>
constexpr int units_per_step(int fm, int fn) {
  return AB == kF8 ? 2 * fm * fn : AB == kF32 ? 16 * fm * fn : 4 * fm * fn;
}

// Last k-slot whose fragments unit u reads.
template <int AB>
constexpr int unit_last_slot(int u, int fm, int fn) {
  return AB == kF8 ? 2 * (u / (fm * fn)) + 1 : AB == kF32 ? u / (4 * fm * fn) : u / (fm * fn);
}

template <int AB, int FM, int FN, int U0, int U1>
__device__ __forceinline__ void mma_units(f32x16 (&acc)[FM][FN], const i32x4 (&fa)[4][FM],
                                          const i32x4 (&fb)[4][FN]) {
#pragma unroll
  for (int u = U0; u < U1; ++u) {
    const int ij = u % (FM * FN);
    const int i = ij / FN, j = ij % FN;
    if constexpr (AB == kBF16) {
      const int s = u / (FM * FN);
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[s][i]),
                                                          __builtin_bit_cast(bf16x8, fb[s][j]),
                                                          acc[i][j], 0, 0, 0);
    } else if constexpr (AB == kF16) {
      const int s = u / (FM * FN);
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fa[s][i]),
                                                         __builtin_bit_cast(f16x8, fb[s][j]),
                                                         acc[i][j], 0, 0, 0);
    } else if constexpr (AB == kF8) {
      const int h = u / (FM * FN);
      const i32x4 a0 = fa[2 * h][i], a1 = fa[2 * h + 1][i];
      const i32x4 b0 = fb[2 * h][j], b1 = fb[2 * h + 1][j];
      const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const i32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      // format code 0 = fp8 E4M3 for both operands; zero scale operands
      // select the unscaled instruction
      acc[i][j] =
          __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, 0, 0, 0, 0);
    } else {
      // Elements are copied to scalars before reinterpretation: hipcc
      // (clang 22) folds __builtin_bit_cast of a vector-element lvalue to
      // element 0.
      const int st = u / (FM * FN);
      const int s = st >> 2, t = st & 3;
      const int av = fa[s][i][t], bv = fb[s][j][t];
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(av), __int_as_float(bv),
                                                       acc[i][j], 0, 0, 0);
    }
  }
}

// Transpose of an (R k-rows) x (one 16-byte chunk of n) block of an
// N-contiguous B into LDS rows indexed by n holding K contiguously.
// in[r] = chunk of row k0 + r.  Column j of the chunk becomes R k-values
// (R*E bytes) stored in LDS row (nrow0 + j) at byte kbyte of the row.
template <int E, int R>
__device__ __forceinline__ void store_nn_block(char *lds_b, const i32x4 (&in)[R], int nrow0,
                                               int kbyte) {
  constexpr int V = 16 / E;     // columns of the chunk
  constexpr int W = R * E / 4;  // 32-bit words per column
#pragma unroll
  for (int j = 0; j < V; ++j) {
    uint32_t o[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
      if constexpr (E == 4) {
        o[w] = (uint32_t)in[w][j];
      } else if constexpr (E == 2) {
        // low or high half of word j/2 of rows 2w and 2w+1
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        o[w] = __builtin_amdgcn_perm((uint32_t)in[2 * w + 1][j >> 1], (uint32_t)in[2 * w][j >> 1], sel);
      } else {
        // byte j%4 of word j/4 of rows 4w .. 4w+3 (selector 0x0c gives 0)
        const uint32_t b = j & 3;
        const uint32_t sel = b | ((4u + b) << 8) | 0x0c0c0000u;
        const uint32_t t0 = __builtin_amdgcn_perm((uint32_t)in[4 * w + 1][j >> 2], (uint32_t)in[4 * w][j >> 2], sel);
        const uint32_t t1 = __builtin_amdgcn_perm((uint32_t)in[4 * w + 3][j >> 2], (uint32_t)in[4 * w + 2][j >> 2], sel);
        o[w] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
      }
    }
    char *dst = lds_b + lds_off(nrow0 + j, kbyte >> 4) + (kbyte & 15);
    if constexpr (W == 8) {
      *(i32x4 *)dst = i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
      *(i32x4 *)(lds_b + lds_off(nrow0 + j, (kbyte >> 4) + 1)) = i32x4{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
    } else if constexpr (W == 4) {
      *(i32x4 *)dst = i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    } else if constexpr (W == 2) {
      *(i32x2 *)dst = i32x2{(int)o[0], (int)o[1]};
    } else {
      *(int *)dst = (int)o[0];
    }
  }
}

// Scheduling hint for a region holding NM MFMAs, NR LDS reads and NV
// global loads: two MFMAs, then the loads and LDS reads, then the other
// MFMAs.  The compiler puts a full LDS wait (lgkmcnt(0)) before a region's
// first MFMA when loop-carried fragments and direct-to-LDS loads are in
// flight; issuing the region's own reads after that MFMA keeps the wait
// from covering them, and they still get most of the region to complete.
template <int NM, int NR, int NV = 0>
__device__ __forceinline__ void interleave() {
  constexpr int lead = NM < 2 ? NM : 2;
  if constexpr (lead > 0) __builtin_amdgcn_sched_group_barrier(0x008, lead, 0);    // MFMAs
  if constexpr (NR > 0) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);        // LDS reads
  if constexpr (NV > 0) __builtin_amdgcn_sched_group_barrier(0x020, NV, 0);        // global loads
  if constexpr (NM > lead) __builtin_amdgcn_sched_group_barrier(0x008, NM - lead, 0);
}

// ---------------------------------------------------------------- kernel

// FULL selects the full-form epilogue (beta * old C, activation); the plain
// one is a separate instantiation so that the main loop's register
// allocation does not carry the larger epilogue.
template <int AB, int CT, bool NT, int BM, int BN, int NW, bool VEC, bool FULL>
__global__ __launch_bounds__(64 * NW) void gemm_mfma_kernel(GemmParams p) {
  constexpr int E = FmtBytes<AB>::value;
  constexpr int CE = FmtBytes<CT>::value;
  constexpr int V = 16 / E;           // elements per 16-byte chunk
  constexpr int BK = kRowBytes / E;   // elements of K per step
  constexpr int NTH = 64 * NW;          // threads; NW waves as a 2 x (NW/2) grid over the tile
  constexpr int WGN = NW / 2;
  constexpr int WTM = BM / 2, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_BYTES = BM * kRowBytes;
  constexpr int STAGE = (BM + BN) * kRowBytes;
  constexpr int AL = BM * 8 / NTH;            // A chunks per thread (= direct loads per wave)
  constexpr int RNN = 8 * BN / NTH;           // NN: k-rows per thread's B block
  constexpr int BL = NT ? BN * 8 / NTH : RNN; // B chunks per thread
  constexpr int U = units_per_step<AB>(FM, FN);
  constexpr int UL = U / 8;                   // units issued after the step's barrier
  constexpr int PRE = AB == kF8 ? 2 : 1;      // k-slots read before a step starts
  static_assert(RNN == 4 || RNN == 8, "NN B blocks of 4 or 8 k-rows, one per thread");
  static_assert(unit_last_slot<AB>(U - UL, FM, FN) == 3, "late units must read slot 3 only");
  static_assert(unit_last_slot<AB>(U / 4 - 1, FM, FN) < PRE, "phase 0 uses preloaded slots");

  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

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

  // Per-lane byte offsets from the problem's base pointers.  The host only
  // selects this kernel when each operand spans less than 4 GiB, so they fit
  // 32 bits.
  // ---- register-path sources (partial K-step, and the element path):
  // thread moves chunk c of rows (tid / 8) + 32 i
  const int c = tid & 7;
  uint32_t a_src[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int64_t r = min64(m0 + (tid >> 3) + (NTH / 8) * i, M - 1);
    a_src[i] = (uint32_t)(r * p.lda * E + c * 16);
  }
  uint32_t b_src[NT ? BL : 1];
  uint32_t nn_src = 0;         // NN: offset of row (RNN nn_kb) of this thread's column chunk
  int nb_valid = 0;            // NN: valid columns in this thread's chunk
  int nn_kb = 0, nn_nc = 0;    // NN: RNN-row k block and n chunk of this thread
  const uint32_t ldb_bytes = (uint32_t)(p.ldb * E);
  if constexpr (NT) {
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int64_t r = min64(n0 + (tid >> 3) + (NTH / 8) * i, N - 1);
      b_src[i] = (uint32_t)(r * p.ldb * E + c * 16);
    }
  } else {
    constexpr int KB = BK / RNN;  // row blocks per K-step; KB * (BN / V) == NTH
    // column chunk fastest: consecutive lanes read consecutive 16 bytes of a B row
    nn_nc = tid % (BN / V);
    nn_kb = tid / (BN / V);
    static_assert(KB * (BN / V) == NTH, "one NN B block per thread");
    const int64_t ncol = n0 + (int64_t)nn_nc * V;
    nb_valid = (int)max64(0, min64(V, N - ncol));
    const int64_t ccol = nb_valid > 0 ? ncol : 0;
    nn_src = (uint32_t)(((int64_t)(nn_kb * RNN) * p.ldb + ccol) * E);
  }

  // ---- direct global->LDS sources (16-byte path, whole K-steps).  Wave w
  // fills rows [w*BM/NW, (w+1)*BM/NW) of the A stage, 8 rows per instruction;
  // lane L lands at position L%8 of row L/8 of its 8-row block, so it loads
  // logical chunk (L%8) ^ swz(row) of that row.
  uint32_t a_dl[VEC ? AL : 1];
  uint32_t b_dl[VEC && NT ? BL : 1];
  if constexpr (VEC) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int row = wave * (BM / NW) + i * 8 + (lane >> 3);
      const int64_t r = min64(m0 + row, M - 1);
      a_dl[i] = (uint32_t)(r * p.lda * E + (((lane & 7) ^ swz(row)) << 4));
    }
    if constexpr (NT) {
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        const int row = wave * (BN / NW) + i * 8 + (lane >> 3);
        const int64_t r = min64(n0 + row, N - 1);
        b_dl[i] = (uint32_t)(r * p.ldb * E + (((lane & 7) ^ swz(row)) << 4));
      }
    }
  }

  i32x4 ra[AL], rb[BL];

  // Issue the direct loads of whole K-step kt into `stage` (A, and B when NT).
  auto issue_direct = [&](int64_t kt, int stage) __attribute__((always_inline)) {
    const int64_t kofs = kt * kRowBytes;
    char *la = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < AL; ++i)
      load16_to_lds(A + kofs + a_dl[i], la + (wave * (BM / NW) + i * 8) * kRowBytes);
    if constexpr (NT) {
#pragma unroll
      for (int i = 0; i < BL; ++i)
        load16_to_lds(B + kofs + b_dl[i], la + A_BYTES + (wave * (BN / NW) + i * 8) * kRowBytes);
    }
  };

  // NN B rows of whole K-step kt into registers: a chunk wholly inside N in
  // one 16-byte load (any element alignment), the chunk that N cuts through
  // (16-bit: one 16-byte load ending at its last valid element when rows
  // hold at least 8 elements, shifted into place when it is stored to LDS;
  // else by elements) and one wholly past N as zeros (it only feeds outputs
  // that are never stored).  A per-lane branch around the loads, or work on
  // the loaded data here, costs the wave its load overlap (4097 x 511 x 1023
  // bf16: 65 us with a word-load branch for the cut chunk, against 19 us at
  // N = 512).
  const bool nn_tail16 = E == 2 && N >= V && N % V != 0;
  auto load_nn_full = [&](int64_t kt) __attribute__((always_inline)) {
    const char *bk = B + kt * BK * p.ldb * E;
#pragma unroll
    for (int r = 0; r < RNN; ++r) {
      const char *q = bk + (nn_src + r * ldb_bytes);
      if constexpr (E == 2) {
        if (N % V == 0) rb[r] = load16(q);  // chunks wholly inside or past N (past: column 0, unused)
        else if (nn_tail16) rb[r] = load16(tail_load_addr(q, nb_valid));
        else rb[r] = load_chunk_elems<E>(q, nb_valid);
      } else {
        rb[r] = nb_valid == V ? load16(q) : load_chunk_elems<E>(q, nb_valid);
      }
    }
  };

  // Register path for any K-step: element loads, zero past K (and past N for NN).
  auto load_regs = [&](int64_t kt) __attribute__((always_inline)) {
    const int64_t kofs = kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int64_t k0 = kt * BK + c * V;
      const int nv = (int)max64(0, min64(V, K - k0));
      const char *q = A + kofs + a_src[i];
      ra[i] = (VEC && nv == V) ? load16(q) : load_chunk_elems<E>(q, nv);
    }
    if constexpr (NT) {
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        const int64_t k0 = kt * BK + c * V;
        const int nv = (int)max64(0, min64(V, K - k0));
        const char *q = B + kofs + b_src[i];
        rb[i] = (VEC && nv == V) ? load16(q) : load_chunk_elems<E>(q, nv);
      }
    } else {
      const char *bk = B + kt * BK * p.ldb * E;
#pragma unroll
      for (int r = 0; r < RNN; ++r) {
        const char *q = bk + (nn_src + r * ldb_bytes);
        const bool krow_ok = kt * BK + nn_kb * RNN + r < K;
        rb[r] = (VEC && nb_valid == V && krow_ok) ? load16(q)
                                                   : load_chunk_elems<E>(q, krow_ok ? nb_valid : 0);
      }
    }
  };

  // `tail`: rb holds load_nn_full's raw loads (the cut chunk still to be
  // shifted into place), not load_regs' finished chunks.
  auto store_nn = [&](int stage, bool tail) __attribute__((always_inline)) {
    if constexpr (!NT) {
      if constexpr (E == 2) {
        if (tail && nn_tail16) {
#pragma unroll
          for (int r = 0; r < RNN; ++r) rb[r] = tail_shift(rb[r], nb_valid);
        }
      }
      store_nn_block<E, RNN>(lds + stage * STAGE + A_BYTES, rb, nn_nc * V, nn_kb * RNN * E);
    }
  };

  auto store_regs = [&](int stage) __attribute__((always_inline)) {
    char *la = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < AL; ++i) *(i32x4 *)(la + lds_off((tid >> 3) + (NTH / 8) * i, c)) = ra[i];
    if constexpr (NT) {
#pragma unroll
      for (int i = 0; i < BL; ++i)
        *(i32x4 *)(la + A_BYTES + lds_off((tid >> 3) + (NTH / 8) * i, c)) = rb[i];
    } else {
      store_nn(stage, false);
    }
  };

  // Fragment addresses: a lane reads row (block base + l32), chunk 2s + g.
  // Block bases are multiples of 32 and each wave's first block a multiple
  // of 64, so swz(base + l32) = swz(l32) ^ (4 if the block index is odd).
  static_assert(WTM % 64 == 0 && WTN % 64 == 0, "wave tiles start on 64-row boundaries");
  int choff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) choff[s] = ((2 * s + g) ^ swz(l32)) << 4;
  const int a_frag = (wm * WTM + l32) * kRowBytes;
  const int b_frag = A_BYTES + (wn * WTN + l32) * kRowBytes;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  i32x4 fa[4][FM], fb[4][FN];
  auto read_slot = [&](int stage, int s) __attribute__((always_inline)) {
    const char *base = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[s][i] = *(const i32x4 *)(base + a_frag + i * 32 * kRowBytes + (choff[s] ^ ((i & 1) << 6)));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[s][j] = *(const i32x4 *)(base + b_frag + j * 32 * kRowBytes + (choff[s] ^ ((j & 1) << 6)));
  };
  // Units of phase q (q < 3) of a K-step.
  auto mma_units_phase = [&](int q) __attribute__((always_inline)) {
    if (q == 0) mma_units<AB, FM, FN, 0, U / 4>(acc, fa, fb);
    else if (q == 1) mma_units<AB, FM, FN, U / 4, U / 2>(acc, fa, fb);
    else mma_units<AB, FM, FN, U / 2, 3 * U / 4>(acc, fa, fb);
  };

  // All LDS writes of this wave (direct and ds_write) done, then the barrier.
  auto stage_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  const int64_t nsteps = (K + BK - 1) / BK;
  const int64_t nfull = K / BK;

  // One K-step on stage `cur`, in four phases of U/4 matrix instructions.
  // The fragments of the first PRE k-slots are already in registers; phase
  // q reads slot PRE + q, so every slot is read at least one phase before
  // the instructions that use it.  The next stage is written
  // in the last phase, well after its global loads were issued; the barrier
  // falls before the last UL instructions, so the first fragment reads of
  // stage `nxt` overlap the step's final instructions.  Scheduling barriers
  // keep the phases apart; group barriers interleave reads and MFMAs.
  // Whole K-steps (!from_regs) issue the next step's global loads inside
  // phases 0 (direct A / NT B) and 1 (NN B into registers).
  constexpr int NV0 = AL + (NT ? BL : 0);
  constexpr int NV1 = NT ? 0 : RNN;
  constexpr int NR = FM + FN;
  auto step_body = [&](int64_t kt, int cur, int nxt, bool from_regs) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (PRE + q < 4) read_slot(cur, PRE + q);
      if (!from_regs && q == 0) issue_direct(kt + 1, nxt);
      if constexpr (!NT) {
        if (!from_regs && q == 1) load_nn_full(kt + 1);
      }
      mma_units_phase(q);
      if (from_regs) {
        if (PRE + q < 4) interleave<U / 4, NR>();
      } else if (q == 0) {
        interleave<U / 4, (PRE < 4 ? NR : 0), NV0>();
      } else if (q == 1) {
        interleave<U / 4, (PRE + 1 < 4 ? NR : 0), NV1>();
      } else {
        if (PRE + q < 4) interleave<U / 4, NR>();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (from_regs)
      store_regs(nxt);
    else
      store_nn(nxt, true);
    mma_units<AB, FM, FN, 3 * U / 4, U - UL>(acc, fa, fb);
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier();
#pragma unroll
    for (int s0 = 0; s0 < PRE; ++s0) read_slot(nxt, s0);
    mma_units<AB, FM, FN, U - UL, U>(acc, fa, fb);
    interleave<UL, PRE * NR>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: step 0 into stage 0
  if (VEC && nfull > 0) {
    issue_direct(0, 0);
    if constexpr (!NT) {
      load_nn_full(0);
      store_nn(0, true);
    }
  } else {
    load_regs(0);
    store_regs(0);
  }
  stage_barrier();
#pragma unroll
  for (int s0 = 0; s0 < PRE; ++s0) read_slot(0, s0);

  int64_t kt = 0;
  if constexpr (VEC) {
    // steady state: the next step is a whole one
    for (; kt + 1 < nfull; ++kt) {
      const int cur = (int)(kt & 1), nxt = cur ^ 1;
      step_body(kt, cur, nxt, false);
    }
  }
  // remaining steps through registers (partial K-step, or the element path)
  for (; kt + 1 < nsteps; ++kt) {
    const int cur = (int)(kt & 1), nxt = cur ^ 1;
    load_regs(kt + 1);
    step_body(kt, cur, nxt, true);
  }
  // last step
  {
    const int cur = (int)(kt & 1);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (PRE + q < 4) read_slot(cur, PRE + q);
      mma_units_phase(q);
    }
    mma_units<AB, FM, FN, 3 * U / 4, U>(acc, fa, fb);
  }

  // ---- epilogue: scale, bias, round once, masked store, staged through
  // LDS (free once every wave has passed this barrier)
  static_assert(NW * 32 * stage_pitch<CT, BN / (NW / 2)>() <= 2 * STAGE, "epilogue staging");
  __syncthreads();
  char *C = (char *)p.C + z * p.strideC * CE;
  if constexpr (FULL) {
    static_assert(NW * 16 * (WTN * 4 + 32) <= 2 * STAGE, "full-form epilogue staging");
    store_tile_ex<CT, FM, FN>(acc, lds + wave * 16 * (WTN * 4 + 32), C, p.ldc, M, N, m0 + wm * WTM,
                              n0 + wn * WTN, p.bias, p.scale, p.beta, p.act, lane);
  } else {
    store_tile_lds<CT, FM, FN>(acc, lds + wave * 32 * stage_pitch<CT, WTN>(), C, p.ldc, M, N,
                               m0 + wm * WTM, n0 + wn * WTN, p.bias, p.scale, lane);
  }
}

template <int AB, int CT, bool NT, int BM, int BN, int NW, bool VEC>
hipError_t launch_one(const GemmParams &p, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.batch;
  if (p.beta != 0.f || p.act != 0)
    hipLaunchKernelGGL((gemm_mfma_kernel<AB, CT, NT, BM, BN, NW, VEC, true>), dim3((unsigned)tiles),
                       dim3(64 * NW), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_mfma_kernel<AB, CT, NT, BM, BN, NW, VEC, false>), dim3((unsigned)tiles),
                       dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

template <int AB, int CT, bool NT, int NW>
hipError_t launch_ring(const GemmParams &p, hipStream_t stream);

template <int AB, int CT, bool NT, int BM, int BN, int TAIL>
hipError_t launch_quad(const GemmParams &p, hipStream_t stream);

template <int AB, int CT, bool NT, int TAIL>
hipError_t launch_quad_deep(const GemmParams &p, hipStream_t stream);

// Whether the 128x128 four-wave tiles take the eight-stage ring: one round
// of tiles (each CU streams its own panels, so seven steps in flight instead
// of three hide more of the loads' latency), the plain epilogue, and at
// least 8 ring steps; `kt` is the K-tail form's tail (0 in the plain form).
// The override's ring=4 / ring=8 pins it either way where it applies.
inline bool quad_deep(const GemmParams &p, int64_t kt) {
  if (p.beta != 0.f || p.act != 0 || (p.K - kt) / 32 < 8) return false;
  const int r = ring_override();
  if (r) return r == 8;
  return ((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch <= device_cu_count();
}

// Whether the four-wave kernel applies to 16-bit inputs: its plain form
// (TAIL = 0) takes an even number, at least 4, of 32-element K-steps with
// whole 16-byte chunks in every row; its K-tail form (kQuadTail) any K whose
// part below the last 64-element boundary short of K (short of K - 64 when
// 64 divides K) holds at least 4 steps, including an NN B whose rows end
// inside a chunk (N >= 8 for that one, so the chunk a row's end cuts through
// has a next k-row to read into).
template <bool NT>
int quad_form(const GemmParams &p, int e) {
  const bool cut = !NT && (p.N * e) % 16 != 0;
  if (!cut && p.K % 64 == 0 && p.K >= 128) return 0;
  const int64_t kt = p.K % 64 ? p.K % 64 : 64;
  if (p.K - kt >= 128 && (!cut || p.N >= 8)) return 4;  // kQuadTail
  return -1;
}

template <int CT, bool NT>
hipError_t launch_quad8(const GemmParams &p, hipStream_t stream);

template <int AB, int CT, bool NT>
hipError_t launch_tile(Tile tile, bool vec, const GemmParams &p, hipStream_t stream) {
  if (vec) {
    switch (tile) {
      case kTile256x256:
      case kTile256x256q:
        // Four-wave kernel (gemm_quad.h): 16-bit inputs, an even number (at
        // least 4) of 32-element K-steps or the K-tail form, the plain or
        // full form.  Chosen for every such 256x256 tile: it measured faster
        // than the ring and two-stage kernels at every shape timed (4096^3
        // NN fp32 out 118.1 -> 102.3 us; 8192x12288x4096 NT 661.6 -> 621.5
        // us; 8192^3 NN 880 -> 765 us).
        if constexpr (AB == kBF16 || AB == kF16) {
          const int form = quad_form<NT>(p, 2);
          if (form == 0) return launch_quad<AB, CT, NT, 256, 256, 0>(p, stream);
          if (form > 0) return launch_quad<AB, CT, NT, 256, 256, 4>(p, stream);
          // an NN B cut inside a chunk that the K-tail form does not take:
          // the two-stage kernel (the ring below loads whole chunks)
          if (!NT && (p.N * 2) % 16 != 0) return launch_one<AB, CT, NT, 256, 256, 8, true>(p, stream);
        }
        // fp8: the four-wave kernel of gemm_quad8.h (an even number, at least
        // 4, of 64-element K-steps; the plain form): 8192^3 NN bf16 out
        // 442 -> 426 us against the eight-wave ring
        if constexpr (AB == kF8) {
          if (p.K % 128 == 0 && p.K >= 256 && p.beta == 0.f && p.act == 0) return launch_quad8<CT, NT>(p, stream);
        }
        [[fallthrough]];
      case kTile256x256r:
        // Four-stage ring kernel (gemm_ring.h) for 16-bit and fp8 inputs and
        // whole 64-byte K-steps; chosen automatically for fp8, and for 16-bit
        // inputs with an N-contiguous B when the four-wave kernel does not
        // apply (with a K-contiguous 16-bit B the two-stage kernel measured
        // faster).
        if constexpr (AB != kF32) {
          if (p.K % (64 / FmtBytes<AB>::value) == 0 &&
              (tile == kTile256x256r || !NT || AB == kF8))
            return launch_ring<AB, CT, NT, 8>(p, stream);
        }
        // the eight-wave two-stage kernel's fp8 fragments do not fit in 256
        // registers per lane; fp8 takes four waves (accumulators in AGPRs)
        if constexpr (AB == kF8) return launch_one<AB, CT, NT, 256, 256, 4, true>(p, stream);
        return launch_one<AB, CT, NT, 256, 256, 8, true>(p, stream);
      case kTile256x128q:
      case kTile128x128q:
        // the four-wave kernel on narrower tiles, in its plain or K-tail form
        // (ragged 4097 x 511 x 1023 NN bf16: 39.6 us on the two-stage kernel)
        if constexpr (AB == kBF16 || AB == kF16) {
          const int form = quad_form<NT>(p, 2);
          if (form == 0) {
            if (tile == kTile256x128q) return launch_quad<AB, CT, NT, 256, 128, 0>(p, stream);
            if (quad_deep(p, 0)) return launch_quad_deep<AB, CT, NT, 0>(p, stream);
            return launch_quad<AB, CT, NT, 128, 128, 0>(p, stream);
          }
          if (form > 0) {
            if (tile == kTile256x128q) return launch_quad<AB, CT, NT, 256, 128, 4>(p, stream);
            if (quad_deep(p, p.K % 64 ? p.K % 64 : 64)) return launch_quad_deep<AB, CT, NT, 4>(p, stream);
            return launch_quad<AB, CT, NT, 128, 128, 4>(p, stream);
          }
        }
        if (tile == kTile256x128q) return launch_one<AB, CT, NT, 256, 128, 4, true>(p, stream);
        return launch_one<AB, CT, NT, 128, 128, 4, true>(p, stream);
      case kTile256x256s2:
        if constexpr (AB == kF8) return launch_one<AB, CT, NT, 256, 256, 4, true>(p, stream);
        return launch_one<AB, CT, NT, 256, 256, 8, true>(p, stream);
      case kTile256x256w4: return launch_one<AB, CT, NT, 256, 256, 4, true>(p, stream);
      case kTile256x128: return launch_one<AB, CT, NT, 256, 128, 4, true>(p, stream);
      default: return launch_one<AB, CT, NT, 128, 128, 4, true>(p, stream);
    }
  }
  return launch_one<AB, CT, NT, 128, 128, 4, false>(p, stream);
}

template <int AB, int CT>
hipError_t launch_layout(bool trans_b, Tile tile, bool vec, const GemmParams &p,
                         hipStream_t stream) {
  return trans_b ? launch_tile<AB, CT, true>(tile, vec, p, stream)
                 : launch_tile<AB, CT, false>(tile, vec, p, stream);
}

}  // namespace gemm_detail
}  // namespace tmm
