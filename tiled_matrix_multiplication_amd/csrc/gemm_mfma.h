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
//     32 consecutive rows and the row-wise writes hit distinct banks (the
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
//     the linear-layer formula of the GEMM page).
//   * Edges: rows past M (columns past N) of A (op(B)) are read from the
//     last valid row, which only feeds outputs that are never stored; the K
//     tail is zero-filled; stores are masked (tiled_matmul's min() bounds).
//   * Tile order: workgroups are spread round-robin over the 8 XCDs, so the
//     tile index is remapped to give each XCD a contiguous run of tiles,
//     grouped 4 tile-rows deep so the run shares A and B panels in that
//     XCD's L2 (devpress notes section 3.7 on tiles versus compute units).
#pragma once

#include "tmm_internal.h"

namespace tmm {
namespace gemm_detail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int F> struct FmtBytes;
template <> struct FmtBytes<kF32> { static constexpr int value = 4; };
template <> struct FmtBytes<kBF16> { static constexpr int value = 2; };
template <> struct FmtBytes<kF16> { static constexpr int value = 2; };
template <> struct FmtBytes<kF8> { static constexpr int value = 1; };

constexpr int kRowBytes = 128;  // bytes of one K-step per tile row
constexpr int kThreads = 256;   // 4 waves
constexpr int kGroupM = 4;      // tile-rows per ordering group

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

// Elements [0, nvalid) of the 16-byte chunk at p (element-aligned); zero past them.
template <int E>
__device__ __forceinline__ i32x4 load_chunk_elems(const char *p, int nvalid) {
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

// One K-step (128 bytes per row) of matrix instructions on fragments read
// from LDS.  fa[s][i] / fb[s][j] hold, for k-slot s = 0..3, the 16-byte
// chunk 2s + (lane / 32) of the lane's A row / B column.  A and B use the
// same slot-to-chunk map, so each instruction pairs equal k indices.
template <int AB, int FM, int FN>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[FM][FN], const i32x4 (&fa)[4][FM],
                                         const i32x4 (&fb)[4][FN]) {
  if constexpr (AB == kBF16) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, fa[s][i]), __builtin_bit_cast(bf16x8, fb[s][j]),
              acc[i][j], 0, 0, 0);
  } else if constexpr (AB == kF16) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8, fa[s][i]), __builtin_bit_cast(f16x8, fb[s][j]),
              acc[i][j], 0, 0, 0);
  } else if constexpr (AB == kF8) {
    // 32x32x64: 32 bytes of K per lane = slots 2h and 2h+1.
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const i32x4 a0 = fa[2 * h][i], a1 = fa[2 * h + 1][i];
          const i32x4 b0 = fb[2 * h][j], b1 = fb[2 * h + 1][j];
          const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          const i32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          // format code 0 = fp8 E4M3 for both operands; zero scale operands
          // select the unscaled instruction
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, 0, 0,
                                                                       0, 0);
        }
  } else {
    // fp32 32x32x2: one float of K per lane; a slot's chunk holds 4 floats.
    // Elements are copied to scalars before reinterpretation: hipcc (clang
    // 22) folds __builtin_bit_cast of a vector-element lvalue to element 0.
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int av = fa[s][i][t], bv = fb[s][j][t];
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__int_as_float(av),
                                                              __int_as_float(bv), acc[i][j], 0, 0,
                                                              0);
          }
  }
}

// Transpose of an (8 k-rows) x (one 16-byte chunk of n) block of an
// N-contiguous B into LDS rows indexed by n holding K contiguously.
// in[r] = chunk of row k0 + r.  Column j of the chunk becomes 8 k-values
// (8*E bytes) stored in LDS row (nrow0 + j) at byte kbyte of the row.
template <int E>
__device__ __forceinline__ void store_nn_block(char *lds_b, const i32x4 (&in)[8], int nrow0,
                                               int kbyte) {
  if constexpr (E == 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      i32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        o[w] = (int)__builtin_amdgcn_perm((uint32_t)in[2 * w + 1][j >> 1],
                                          (uint32_t)in[2 * w][j >> 1], sel);
      const int row = nrow0 + j;
      *(i32x4 *)(lds_b + lds_off(row, kbyte >> 4)) = o;
    }
  } else if constexpr (E == 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int wd = j >> 2, sh = 8 * (j & 3);
      uint32_t o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) v |= (((uint32_t)in[4 * h + b][wd] >> sh) & 0xffu) << (8 * b);
        o[h] = v;
      }
      const int row = nrow0 + j;
      *(i32x2 *)(lds_b + lds_off(row, kbyte >> 4) + (kbyte & 15)) = i32x2{(int)o[0], (int)o[1]};
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = nrow0 + j;
      const i32x4 o0 = {in[0][j], in[1][j], in[2][j], in[3][j]};
      const i32x4 o1 = {in[4][j], in[5][j], in[6][j], in[7][j]};
      *(i32x4 *)(lds_b + lds_off(row, kbyte >> 4)) = o0;
      *(i32x4 *)(lds_b + lds_off(row, (kbyte >> 4) + 1)) = o1;
    }
  }
}

// ---------------------------------------------------------------- kernel

template <int AB, int CT, bool NT, int BM, int BN, bool VEC>
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmParams p) {
  constexpr int E = FmtBytes<AB>::value;
  constexpr int CE = FmtBytes<CT>::value;
  constexpr int V = 16 / E;           // elements per 16-byte chunk
  constexpr int BK = kRowBytes / E;   // elements of K per step
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_BYTES = BM * kRowBytes;
  constexpr int STAGE = (BM + BN) * kRowBytes;
  constexpr int AL = BM / 32;                 // A chunks per thread
  constexpr int BL = NT ? BN / 32 : 8;        // B chunks per thread
  static_assert(BN <= kThreads, "one N-contiguous B block per thread");

  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
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

  // ---- per-thread global source addresses
  const int c = tid & 7;  // chunk of a K-contiguous row this thread moves
  const char *a_src[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int64_t r = min64(m0 + (tid >> 3) + 32 * i, M - 1);
    a_src[i] = A + (r * p.lda) * E + c * 16;
  }
  const char *b_src[BL];
  int nb_valid = 0;            // NN: valid columns in this thread's chunk
  int nn_kb = 0, nn_nc = 0;    // NN: 8-row k block and n chunk of this thread
  if constexpr (NT) {
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int64_t r = min64(n0 + (tid >> 3) + 32 * i, N - 1);
      b_src[i] = B + (r * p.ldb) * E + c * 16;
    }
  } else {
    constexpr int KB = BK / 8;  // 8-row blocks per K-step
    nn_kb = tid % KB;
    nn_nc = tid / KB;
    const int64_t ncol = n0 + (int64_t)nn_nc * V;
    nb_valid = (tid < BN) ? (int)max64(0, min64(V, N - ncol)) : 0;
    const int64_t ccol = nb_valid > 0 ? ncol : 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) b_src[r] = B + ((int64_t)(nn_kb * 8 + r) * p.ldb + ccol) * E;
  }

  i32x4 ra[AL], rb[BL];

  // Global -> registers for K-step kt.  `full`: the whole step lies inside K.
  auto load_step = [&](int64_t kt, bool full) {
    const int64_t kofs = kt * kRowBytes;  // byte offset along a K-contiguous row
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const char *q = a_src[i] + kofs;
      if (VEC && full) {
        ra[i] = load16(q);
      } else {
        const int64_t k0 = kt * BK + c * V;
        const int nv = (int)max64(0, min64(V, K - k0));
        ra[i] = (VEC && nv == V) ? load16(q) : load_chunk_elems<E>(q, nv);
      }
    }
    if constexpr (NT) {
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        const char *q = b_src[i] + kofs;
        if (VEC && full) {
          rb[i] = load16(q);
        } else {
          const int64_t k0 = kt * BK + c * V;
          const int nv = (int)max64(0, min64(V, K - k0));
          rb[i] = (VEC && nv == V) ? load16(q) : load_chunk_elems<E>(q, nv);
        }
      }
    } else {
      const int64_t rofs = kt * BK * p.ldb * E;  // K-step kt starts BK rows down
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const char *q = b_src[r] + rofs;
        const bool krow_ok = full || (kt * BK + nn_kb * 8 + r < K);
        if (VEC && nb_valid == V && krow_ok)
          rb[r] = load16(q);
        else
          rb[r] = load_chunk_elems<E>(q, krow_ok ? nb_valid : 0);
      }
    }
  };

  // Registers -> LDS stage.
  auto store_step = [&](int stage) {
    char *la = lds + stage * STAGE;
    char *lb = la + A_BYTES;
#pragma unroll
    for (int i = 0; i < AL; ++i) *(i32x4 *)(la + lds_off((tid >> 3) + 32 * i, c)) = ra[i];
    if constexpr (NT) {
#pragma unroll
      for (int i = 0; i < BL; ++i) *(i32x4 *)(lb + lds_off((tid >> 3) + 32 * i, c)) = rb[i];
    } else {
      if (tid < BN) store_nn_block<E>(lb, rb, nn_nc * V, nn_kb * 8 * E);
    }
  };

  // Fragment addresses: a lane reads row (block base + l32), chunk 2s + g.
  // Block bases are multiples of 32, so swz(row) = swz(l32).
  int choff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) choff[s] = ((2 * s + g) ^ swz(l32)) << 4;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute_step = [&](int stage) {
    const char *la = lds + stage * STAGE;
    const char *lb = la + A_BYTES;
    i32x4 fa[4][FM], fb[4][FN];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[s][i] = *(const i32x4 *)(la + (wm * WTM + i * 32 + l32) * kRowBytes + choff[s]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[s][j] = *(const i32x4 *)(lb + (wn * WTN + j * 32 + l32) * kRowBytes + choff[s]);
    }
    mma_step<AB, FM, FN>(acc, fa, fb);
  };

  const int64_t nsteps = (K + BK - 1) / BK;
  const int64_t nfull = K / BK;
  load_step(0, nfull > 0);
  store_step(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nsteps; ++kt) {
    const bool more = kt + 1 < nsteps;
    if (more) load_step(kt + 1, kt + 1 < nfull);
    compute_step((int)(kt & 1));
    if (more) store_step((int)((kt + 1) & 1));
    __syncthreads();
  }

  // ---- epilogue: scale, bias, round once, masked store
  char *C = (char *)p.C + z * p.strideC * CE;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = n0 + wn * WTN + j * 32 + l32;
    if (col >= N) continue;
    const float bv = p.bias ? p.bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < M) {
          float v = acc[i][j][r];
          if constexpr (AB == kF8) v *= p.scale;
          v += bv;
          store_out<CT>(C, row * p.ldc + col, v);
        }
      }
    }
  }
}

template <int AB, int CT, bool NT, int BM, int BN, bool VEC>
hipError_t launch_one(const GemmParams &p, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.batch;
  hipLaunchKernelGGL((gemm_mfma_kernel<AB, CT, NT, BM, BN, VEC>), dim3((unsigned)tiles),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int AB, int CT, bool NT>
hipError_t launch_tile(Tile tile, bool vec, const GemmParams &p, hipStream_t stream) {
  if (vec) {
    switch (tile) {
      case kTile256x256: return launch_one<AB, CT, NT, 256, 256, true>(p, stream);
      case kTile256x128: return launch_one<AB, CT, NT, 256, 128, true>(p, stream);
      default: return launch_one<AB, CT, NT, 128, 128, true>(p, stream);
    }
  }
  return launch_one<AB, CT, NT, 128, 128, false>(p, stream);
}

template <int AB, int CT>
hipError_t launch_layout(bool trans_b, Tile tile, bool vec, const GemmParams &p,
                         hipStream_t stream) {
  return trans_b ? launch_tile<AB, CT, true>(tile, vec, p, stream)
                 : launch_tile<AB, CT, false>(tile, vec, p, stream);
}

}  // namespace gemm_detail
}  // namespace tmm
