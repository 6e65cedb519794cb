// Batched C[z] = A[z] . B[z]^T for a short K (64 or 128 16-bit elements)
// over whole 256x256 tiles with a 16-bit output: the shape of attention's
// scores S = Q . K^T (batch x heads problems of 2048 x 2048 at head size
// 128, "GEMM to FlashAttention" page, attention formula and
// attention_standard listing).  Each tile is a few microseconds of matrix
// work and then 128 KiB of stores, so the product is bound by its writes
// (the N x N score traffic the page singles out), and what matters is that
// the stores never wait for the loads and matrix work of the next tile.
//
// One 512-lane workgroup per CU walks tiles bid, bid + G, ... (G a multiple
// of 8, so a tile runs on the XCD its index remap assumes):
//   * the whole K of a tile fits in LDS at once: A (256 rows) and B (256
//     rows) of K*2 bytes each, moved with 16-byte direct global->LDS loads
//     (16 or 8 per wave), chunk c of row r at c ^ f(r) (f(r) = r mod 16 for
//     256-byte rows; (r / 2) mod 8 for 128-byte rows, whose odd rows sit on
//     the other half of the banks), so 16 consecutive rows read at one
//     chunk hit distinct banks;
//   * eight waves own 128x64 blocks of the tile as 4x2 32x32 accumulators
//     (v_mfma_f32_32x32x16 over K/16 slices), as in the two-stage kernel;
//   * after the last matrix instruction and a barrier, the waves issue the
//     next tile's direct loads into the operand area, then stage and store
//     the first 32-row band of their block (band_out below, through each
//     wave's own 4 KiB past the operands: 160 KiB in all at K = 128) and
//     keep the other three bands as packed 16-bit values (48 registers);
//     those go out during the next tile's matrix work, one band after each
//     quarter of its K slices, so that their staging runs while the matrix
//     pipe is busy instead of after it;
//   * a wave then waits with vmcnt(4), its first band's stores: the loads,
//     issued before them, are complete (and so are the previous tile's
//     bands, issued before the loads), while these stores may still be
//     draining.  This is why the loads are written as assembly (untracked
//     by the compiler, which would otherwise wait for everything) and why
//     the host sends only whole tiles here: every wave issues exactly 4
//     stores per band.  The loads take 32-bit offsets from a wave-uniform
//     base (the host keeps lda and ldb below 2^22).
// No bias, no scale (the plain 16-bit form); anything else takes the
// general kernels.
#include "gemm_ring.h"

namespace tmm {
namespace gemm_detail {
namespace {

// 16-byte direct global->LDS load of base + off (base wave-uniform, off this
// lane's 32-bit byte offset); lane L's 16 bytes land at LDS byte m0 + 16 L.
__device__ __forceinline__ void dma16_off(const char *base, uint32_t off, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(m0) : "memory");
}

template <int RB>
__device__ __forceinline__ int sk_swz(int row) {
  return RB == 256 ? (row & 15) : ((row >> 1) & 7);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to two 16-bit values of format F, nearest-even, lo in the low
// half (one packed conversion instruction on gfx950; the same bits as
// out_bits for each).
template <int F>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (F == kBF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

// Epilogue staging of one 32x64 band of a wave's block, held transposed:
// staging row n (output column n of the band) holds the band's 32 rows in
// 8-byte units (4 rows each), 64 bytes a row, unit u at position
// u ^ f(n / 4 mod 8).  f maps column quads 0-3 to even and 4-7 to odd
// positions, and f(t), f(t + 2), f(t + 4), f(t + 6) hold no two values
// that differ only in bit 0.  Byte offset mod 256 is 64 (n mod 4) + 8
// (u ^ f): a write instruction (32 consecutive columns at units u and
// u + 1) and a transposing read (per 16 lanes 4 columns of each of 4
// quads, t fixed, at one unit; the group it shares banks with at the
// adjacent unit) then touch distinct banks whether the hardware serves
// lanes 0-31 together or lanes 0-15 with 32-47.
__device__ __forceinline__ int tr_swz(int m) { return ((m & 3) << 1) ^ (3 * ((m >> 2) & 1)); }
__device__ __forceinline__ int tr_pos(int n, int u) { return n * 64 + ((u ^ tr_swz((n >> 2) & 7)) << 3); }

// Stores one 32x64 band (rows row0 .., columns col0 .. col0 + 63) of 16-bit
// values from its packed form w[j][q]: lane (l32, g) holds, for column
// 32 j + l32 and row group q, rows 8 q + 4 g .. + 3 as one 8-byte unit (two
// words), written to the wave's 4 KiB staging area st in one instruction
// per unit (4 per 32x32 block instead of 16 two-byte writes).  The
// transposing read ds_read_b64_tr_b16 gives lane j of a 16-lane group
// element j % 4 of the units addressed by lanes j / 4, 4 + j / 4, 8 + j / 4
// and 12 + j / 4; with lane 4 k + a addressing column c0 + 8 a + 4 t + k at
// the unit of rows R0 .. R0 + 3, lane 4 a + b receives row R0 + b, columns
// c0 + 8 a + 4 t .. + 3, and two reads (t = 0, 1) make its 16-byte row
// piece.  One store instruction then writes 8 whole 128-byte rows (two
// groups per 4 rows, 32 columns each).  Whole tiles only, C and its pitch
// 16-byte aligned (the host's conditions for this kernel).
__device__ __forceinline__ void band_out(const uint32_t (&w)[2][4][2], char *st, char *C, int64_t ldc,
                                         int64_t row0, int64_t col0, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  const int G = lane >> 4, i16 = lane & 15;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(i32x2 *)(st + tr_pos(32 * j + l32, 2 * q + g)) = i32x2{(int)w[j][q][0], (int)w[j][q][1]};
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r0 = 8 * s + 4 * ((G & 1) ^ (G >> 1)), c0 = 32 * (G >> 1);
    i32x2 h[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      h[t] = __builtin_bit_cast(
          i32x2, lds_read_tr16(st + tr_pos(c0 + 8 * (i16 & 3) + 4 * t + (i16 >> 2), r0 >> 2)));
    const i32x4 v = {h[0][0], h[0][1], h[1][0], h[1][1]};
    char *dst = C + ((row0 + r0 + (i16 & 3)) * ldc + col0 + c0 + 8 * (i16 >> 2)) * 2;
    __builtin_nontemporal_store(v, (i32x4 *)dst);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the staging area is written again
  __builtin_amdgcn_wave_barrier();
}

// The packed form of a band held in accumulators a[0..1] (accumulator
// r = 4 q + e of lane (l32, g): row 8 q + 4 g + e, column 32 j + l32).
template <int CT>
__device__ __forceinline__ void pack_band(const f32x16 (&a)[2], uint32_t (&w)[2][4][2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[j][q][0] = pack2<CT>(a[j][4 * q], a[j][4 * q + 1]);
      w[j][q][1] = pack2<CT>(a[j][4 * q + 2], a[j][4 * q + 3]);
    }
}

template <int AB, int KE>
__global__ __launch_bounds__(512, 1) void gemm_short_k_kernel(GemmParams p) {
  constexpr int E = 2;
  constexpr int CT = AB;                          // 16-bit output of the input's type
  constexpr int RB = KE * E;                      // bytes of one operand row: 128 or 256
  constexpr int CPR = RB / 16;                    // 16-byte chunks per row
  constexpr int BM = 256, BN = 256, NW = 8;
  constexpr int FM = 4, FN = 2, WTM = 128, WTN = 64;
  constexpr int A_BYTES = BM * RB;
  constexpr int OPS = (BM + BN) * RB;             // operand area
  constexpr int STG = 64 * 64;                    // one wave's staging area (a transposed 32x64 band)
  constexpr int RPL = 1024 / RB;                  // rows per direct-load instruction
  constexpr int LOADS = OPS / 1024 / NW;          // direct loads per wave per tile
  constexpr int SLICES = KE / 16;
  static_assert(KE == 64 || KE == 128, "short-K kernel: K = 64 or 128");
  static_assert(LOADS * RPL * NW == BM + BN, "direct-load geometry");
  static_assert(FN == 2 && WTN == 64 && CT != kF32, "epilogue geometry: 32x64 bands of 16-bit values");
  static_assert(OPS + NW * STG <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(16))) char lds[OPS + NW * STG];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / 4, wn = wave % 4;
  const int g = lane >> 5, l32 = lane & 31;

  const int64_t M = p.M, N = p.N;
  const int64_t tiles_m = M / BM, tiles_n = N / BN;
  const int64_t per = tiles_m * tiles_n;
  const int64_t total = per * p.batch;

  const uint32_t lds0 = lds_addr(lds);

  auto tile_of = [&](int64_t t, int64_t &z, int64_t &m0, int64_t &n0) __attribute__((always_inline)) {
    int64_t pid = remap_xcd(t, total);
    z = pid / per;
    pid -= z * per;
    int64_t tm, tn;
    group_order(pid, tiles_m, tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
  };

  auto issue = [&](int64_t t) __attribute__((always_inline)) {
    int64_t z, m0, n0;
    tile_of(t, z, m0, n0);
    const char *A = (const char *)p.A + (z * p.strideA + m0 * p.lda) * E;
    const char *B = (const char *)p.B + (z * p.strideB + n0 * p.ldb) * E;
    // This lane's part of load i: operand row (of the 512 A then B rows)
    // wave * LOADS * RPL + i * RPL + lane / CPR, LDS position lane % CPR,
    // which holds logical chunk (lane % CPR) ^ f(row).  The offsets are
    // recomputed for every tile (cheap) rather than kept in 16 registers
    // across the loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lpos = ln % CPR;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int first = (wave * LOADS + i) * RPL;   // wave-uniform
      const int row = first + ln / CPR;
      const int chunk = lpos ^ sk_swz<RB>(row);
      if (first < BM)
        dma16_off(A, (uint32_t)(row * (uint32_t)(p.lda * E)) + chunk * 16, lds0 + first * RB);
      else
        dma16_off(B, (uint32_t)((row - BM) * (uint32_t)(p.ldb * E)) + chunk * 16, lds0 + first * RB);
    }
  };

  int64_t t = blockIdx.x;
  if (t >= total) return;
  // bands FM - HOLD .. FM - 1 of the previous tile, packed, stored during this tile's slices
  constexpr int HOLD = 3;
  static_assert(HOLD < FM && SLICES % (HOLD + 1) == 0, "held bands");
  uint32_t pk[HOLD][2][4][2];
  char *pC = nullptr;
  int64_t prow0 = 0, pcol0 = 0;
  bool have_prev = false;
  char *const st = lds + OPS + wave * STG;
  issue(t);
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  __syncthreads();

  for (;;) {
    int64_t z, m0, n0;
    tile_of(t, z, m0, n0);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
    for (int s = 0; s < SLICES; ++s) {
      i32x4 fa[FM], fb[FN];
      const int chunk = 2 * s + g;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WTM + i * 32 + l32;
        fa[i] = *(const i32x4 *)(lds + row * RB + ((chunk ^ sk_swz<RB>(row)) << 4));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WTN + j * 32 + l32;
        fb[j] = *(const i32x4 *)(lds + A_BYTES + row * RB + ((chunk ^ sk_swz<RB>(row)) << 4));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (AB == kBF16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[j]), acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, fa[i]), __builtin_bit_cast(f16x8, fb[j]), acc[i][j], 0, 0, 0);
        }
      constexpr int SPB = SLICES / (HOLD + 1);   // slices per held band
      if ((s + 1) % SPB == 0 && (s + 1) / SPB <= HOLD) {
        const int h = (s + 1) / SPB - 1;         // held band h: band FM - HOLD + h of the previous tile
        if (have_prev) band_out(pk[h], st, pC, p.ldc, prow0 + 32 * (FM - HOLD + h), pcol0, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // Every wave's operand reads are done: the area takes the next tile.
    __syncthreads();
    const int64_t next = t + gridDim.x;
    const bool more = next < total;
    if (more) issue(next);

    char *C = (char *)p.C + z * p.strideC * E;
#pragma unroll
    for (int b = 0; b < FM - HOLD; ++b) {
      uint32_t w0[2][4][2];
      pack_band<CT>(acc[b], w0);
      band_out(w0, st, C, p.ldc, m0 + wm * WTM + 32 * b, n0 + wn * WTN, lane);
    }
#pragma unroll
    for (int h = 0; h < HOLD; ++h) pack_band<CT>(acc[FM - HOLD + h], pk[h]);
    pC = C;
    prow0 = m0 + wm * WTM;
    pcol0 = n0 + wn * WTN;
    have_prev = true;
    if (!more) {
#pragma unroll
      for (int h = 0; h < HOLD; ++h) band_out(pk[h], st, pC, p.ldc, prow0 + 32 * (FM - HOLD + h), pcol0, lane);
      break;
    }
    // In issue order: the previous tile's held bands, this tile's loads,
    // this tile's first bands: with their stores outstanding the loads are in.
    __builtin_amdgcn_s_waitcnt(vm_wait(4 * (FM - HOLD)));
    __syncthreads();
    t = next;
  }
}

template <int AB>
hipError_t launch_ab(const GemmParams &p, unsigned grid, hipStream_t stream) {
  if (p.K == 128)
    hipLaunchKernelGGL((gemm_short_k_kernel<AB, 128>), dim3(grid), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_short_k_kernel<AB, 64>), dim3(grid), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace gemm_detail

hipError_t launch_gemm_short_k(Fmt ab, const GemmParams &p, unsigned grid, hipStream_t stream) {
  if (grid == 0 || grid % 8 != 0) return hipErrorInvalidValue;
  if (ab == kBF16) return gemm_detail::launch_ab<kBF16>(p, grid, stream);
  if (ab == kF16) return gemm_detail::launch_ab<kF16>(p, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace tmm
