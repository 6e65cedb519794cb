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
//     next tile's direct loads into the operand area and only then stage
//     and store this tile (store_tile_tr below, through each wave's own
//     4 KiB past the operands: 160 KiB in all at K = 128), so the loads are
//     ahead of the stores in the memory pipeline;
//   * a wave then waits with vmcnt(number of its stores): the loads, issued
//     first, are complete while the stores may still be draining, and the
//     next tile's matrix work overlaps them.  This is why the loads are
//     written as assembly (untracked by the compiler, which would otherwise
//     wait for everything) and why the host sends only whole tiles here:
//     every wave issues exactly FM * 4 stores per tile.
// No bias, no scale (the plain 16-bit form); anything else takes the
// general kernels.
#include "gemm_ring.h"

namespace tmm {
namespace gemm_detail {
namespace {

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

// Stores a wave's FM x 2 accumulator blocks (rows row0 + 32 i + ..., columns
// col0 .. col0 + 63) as 16-bit values, one 32x64 band at a time through the
// wave's own 4 KiB of LDS at st.  Lane (l32, g) writes, for each 4-row group
// of its column, the four values as one 8-byte unit (4 writes per block
// instead of 16 two-byte writes).  The transposing read ds_read_b64_tr_b16
// gives lane j of a 16-lane group element j % 4 of the units addressed by
// lanes j / 4, 4 + j / 4, 8 + j / 4 and 12 + j / 4; with lane 4 k + a
// addressing column c0 + 8 a + 4 t + k at the unit of rows R0 .. R0 + 3,
// lane 4 a + b receives row R0 + b, columns c0 + 8 a + 4 t .. + 3, and two
// reads (t = 0, 1) make its 16-byte row piece.  One store instruction then
// writes 8 whole 128-byte rows (two groups per 4 rows, 32 columns each), as
// a row-major staging would, FM * 4 stores per wave.  Whole tiles only, C
// and its pitch 16-byte aligned (the host's conditions for this kernel).
template <int CT, int FM>
__device__ __forceinline__ void store_tile_tr(const f32x16 (&acc)[FM][2], char *st, char *C, int64_t ldc,
                                              int64_t row0, int64_t col0, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  const int G = lane >> 4, i16 = lane & 15;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // accumulator r = 4 q + e: row 8 q + 4 g + e of the band, column 32 j + l32
        const f32x16 &a = acc[i][j];
        const uint32_t w0 = pack2<CT>(a[4 * q], a[4 * q + 1]);
        const uint32_t w1 = pack2<CT>(a[4 * q + 2], a[4 * q + 3]);
        *(i32x2 *)(st + tr_pos(32 * j + l32, 2 * q + g)) = i32x2{(int)w0, (int)w1};
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // groups 0 and 3 take rows R0 = 8 s .. + 3, groups 1 and 2 the next four
      const int r0 = 8 * s + 4 * ((G & 1) ^ (G >> 1)), c0 = 32 * (G >> 1);
      i32x2 h[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        h[t] = __builtin_bit_cast(
            i32x2, lds_read_tr16(st + tr_pos(c0 + 8 * (i16 & 3) + 4 * t + (i16 >> 2), r0 >> 2)));
      const i32x4 v = {h[0][0], h[0][1], h[1][0], h[1][1]};
      char *dst = C + ((row0 + i * 32 + r0 + (i16 & 3)) * ldc + col0 + c0 + 8 * (i16 >> 2)) * 2;
      __builtin_nontemporal_store(v, (i32x4 *)dst);   // written once, not read back here
    }
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
  constexpr int NSTORE = FM * (32 * (WTN * 2 / 16) / 64);  // store instructions per wave per tile
  static_assert(KE == 64 || KE == 128, "short-K kernel: K = 64 or 128");
  static_assert(LOADS * RPL * NW == BM + BN, "direct-load geometry");
  static_assert(NSTORE <= 63, "vmcnt range");
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
  // This lane's part of each direct load: operand row (of the 512 A then B
  // rows) wave * LOADS * RPL + i * RPL + lane / CPR, LDS position lane % CPR,
  // which holds logical chunk (lane % CPR) ^ f(row).
  const int pos = lane % CPR;

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
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int first = (wave * LOADS + i) * RPL;   // wave-uniform
      const int row = first + lane / CPR;
      const int chunk = pos ^ sk_swz<RB>(row);
      const char *src = row < BM ? A + ((int64_t)row * p.lda * E + chunk * 16)
                                 : B + ((int64_t)(row - BM) * p.ldb * E + chunk * 16);
      dma16(src, lds0 + first * RB);
    }
  };

  int64_t t = blockIdx.x;
  if (t >= total) return;
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
    }

    // Every wave's operand reads are done: the area takes the next tile.
    __syncthreads();
    const int64_t next = t + gridDim.x;
    const bool more = next < total;
    if (more) issue(next);

    char *C = (char *)p.C + z * p.strideC * E;
    store_tile_tr<CT, FM>(acc, lds + OPS + wave * STG, C, p.ldc, m0 + wm * WTM, n0 + wn * WTN, lane);
    if (!more) break;
    // The loads were issued before this wave's NSTORE stores: with at most
    // NSTORE operations outstanding they are complete.
    __builtin_amdgcn_s_waitcnt(vm_wait(NSTORE));
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
