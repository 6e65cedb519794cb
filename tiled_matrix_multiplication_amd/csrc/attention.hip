// Fused attention forward on gfx950 matrix cores, one head per batch entry:
//
//   O[z] = softmax(scale * Q[z] . K[z]^T) . V[z]     (softmax over keys)
//
// the attention of the "GEMM to FlashAttention" page (attention formula and
// attention_standard listing), evaluated the way its
// flash_attention_simplified listing and the Lecture 27 online-softmax slide
// describe: key blocks stream through the chip, each query row keeps a
// running maximum m and exp-sum l, earlier partial outputs are rescaled by
// exp(m_old - m_new), and the Nq x Nk score matrix never reaches memory.
//
// Layout of the work (fp16 or bf16 inputs, fp32 accumulation, head size D =
// 64 or 128):
//   * a workgroup is 4 waves x 32 queries; key blocks of 64 rows of K and of
//     V move global->LDS with 16-byte direct loads into two stages (one
//     block ahead, one barrier per block);
//   * scores are formed transposed, S^T = K . Q^T (K fragments from LDS as
//     the first operand, the wave's Q fragments, loaded once, as the
//     second), so every lane owns one query: its 32 scores of a 32-key block
//     sit in its registers (16) and in lane^32's (16), and the row maximum
//     and exp-sum need one cross-lane exchange;
//   * the output is accumulated transposed too, O^T += V^T . P^T, so a
//     lane's accumulators all belong to its own query and the rescaling by
//     exp(m_old - m_new) is a per-lane multiply.  The weights P (rounded to
//     the input type) are the second operand straight from the score
//     registers; V^T comes from the LDS with the gfx950 transposing read
//     ds_read_b64_tr_b16 (4 consecutive keys of one column per lane).  Both
//     operands use the same order of keys within an instruction, so any
//     order is right;
//   * exponentials are base 2 of log2(e)-prescaled scores (v_exp_f32);
//     keys past Nk score -inf; the last step divides by l and stores.
#include <stdint.h>

#include <type_traits>

#include "tmm_internal.h"

namespace tmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;           // waves per workgroup
constexpr int kQw = 32;             // queries per wave
constexpr int kBQ = kWaves * kQw;   // queries per workgroup
constexpr int kBK = 64;             // keys per block (step)

// 16-byte direct global->LDS load of base + off (off: this lane's 32-bit
// byte offset, base: wave-uniform); lane L's 16 bytes land at LDS byte
// address m0 + 16 L.  From assembly, so the compiler does not track it; the
// kernel waits for these loads itself before each barrier and at exit.
__device__ __forceinline__ void dma16(const char *base, uint32_t off, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(m0)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const char *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

__device__ __forceinline__ s16x4 lds_read_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(__attribute__((address_space(3))) char *)p);
}

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// Workgroups go to XCD (id mod 8): give XCD x a contiguous run of blocks so
// the query blocks of one head share that XCD's L2 for K and V.
__device__ __forceinline__ int64_t remap_xcd(int64_t pid, int64_t n) {
  const int64_t per = n >> 3;
  if (pid >= (per << 3)) return pid;
  return (pid & 7) * per + (pid >> 3);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to two 16-bit values of format F, nearest-even (one packed
// conversion instruction on gfx950), lo in the low half.
template <int F>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (F == kBF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

// LDS swizzles.  K tile: the score fragments read 32 consecutive rows at one
// chunk, so chunk c of row r sits at c ^ (r mod CPR).  V tile: the
// transposing reads of 32 lanes take 4 consecutive rows x 4 chunks (two
// 16-lane halves, 2 chunks each).  With 256-byte rows (D = 128) every row
// spans all 64 banks, so the 4 rows must land on 4 disjoint 64-byte bank
// groups: chunk c of row r sits at c ^ 4 (r mod 4) (c ^ 2 (r mod 4) gave
// two rows the same banks: SQ_LDS_BANK_CONFLICT was 32 % of
// SQ_LDS_IDX_ACTIVE).  With 128-byte rows (D = 64) odd rows already sit on
// the other half of the banks and c ^ 2 (r mod 4) separates the rest.
template <int CPR>
__device__ __forceinline__ int kswz(int row) { return row & (CPR - 1); }
template <int CPR>
__device__ __forceinline__ int vswz(int row) { return (CPR >= 16 ? 4 : 2) * (row & 3); }

// Two waves per SIMD (two workgroups per CU, 64 KiB of LDS each): at most
// 256 registers per lane.
template <int IT, int OT, int D>
__global__ __launch_bounds__(64 * kWaves, 2) void attn_fwd_kernel(AttnParams p) {
  constexpr int E = 2;                    // input bytes
  constexpr int OE = OT == kF32 ? 4 : 2;  // output bytes
  constexpr int RB = D * E;               // bytes of one K / V row
  constexpr int CPR = RB / 16;            // 16-byte chunks per row
  constexpr int TILE = kBK * RB;          // one K or V block
  constexpr int STAGE = 2 * TILE;         // K block, then V block
  constexpr int DS = D / 16;              // k-slices of the score contraction
  constexpr int DB = D / 32;              // 32-column blocks of O
  constexpr int RPI = 64 / CPR;           // rows per direct load
  constexpr int LPT = kBK / RPI / kWaves; // direct loads per wave per tile
  static_assert((D == 64 || D == 128) && LPT >= 1 && CPR >= 8, "attention geometry");

  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int G = lane >> 4, q16 = lane & 15;

  const int64_t Nq = p.Nq, Nk = p.Nk;
  const int64_t qblocks = (Nq + kBQ - 1) / kBQ;
  const int64_t bid = remap_xcd(blockIdx.x, (int64_t)gridDim.x);
  const int64_t z = bid / qblocks;
  const int64_t q0 = (bid - z * qblocks) * kBQ + wave * kQw;
  const char *Qz = (const char *)p.Q + z * p.strideQ * E;
  const char *Kz = (const char *)p.K + z * p.strideK * E;
  const char *Vz = (const char *)p.V + z * p.strideV * E;

  // Q fragments (second operand of S^T = K Q^T), slice c: lane (query
  // q0 + l32, g) holds Q[q][16 c + 8 g .. +7].  Rows past Nq repeat the last
  // query; their outputs are not stored.  A negative scale is moved onto Q
  // (flipping sign bits is exact), so the kernel's scale c is >= 0 and the
  // largest scaled score is c times the largest raw score.
  const bool neg = p.scale_log2 < 0.f;
  const float c2 = neg ? -p.scale_log2 : p.scale_log2;   // log2(e) * |scale|
  i32x4 qf[DS];
  {
    const int64_t qrow = min64(q0 + l32, Nq - 1);
    const int flip = neg ? (int)0x80008000u : 0;
#pragma unroll
    for (int c = 0; c < DS; ++c) {
      qf[c] = *(const i32x4 *)(Qz + (qrow * p.ldq + 16 * c + 8 * g) * E);
#pragma unroll
      for (int w = 0; w < 4; ++w) qf[c][w] ^= flip;
    }
  }

  // Direct loads of key block kb into stage st: instruction i of wave w
  // fills rows (w LPT + i) RPI .. +RPI-1 of the K and of the V tile; lane L
  // lands at row + L/CPR, position L%CPR.  Byte offsets within a block are
  // 32-bit per lane (rows < 64, ld <= 2^24 elements); the block's base
  // address is wave-uniform.  In the last, partial block rows past Nk repeat
  // the last key (their weights are set to 0).
  const uint32_t lds0 = lds_addr(lds);
  const int pos = lane % CPR;
  uint32_t koff[LPT], voff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int row = (wave * LPT + i) * RPI + lane / CPR;
    koff[i] = (uint32_t)(row * p.ldk * E) + ((pos ^ kswz<CPR>(row)) << 4);
    voff[i] = (uint32_t)(row * p.ldv * E) + ((pos ^ vswz<CPR>(row)) << 4);
  }
  auto issue = [&](int64_t kb, int st) __attribute__((always_inline)) {
    const char *kbase = Kz + kb * kBK * p.ldk * E;
    const char *vbase = Vz + kb * kBK * p.ldv * E;
    const int64_t left = Nk - kb * kBK;   // keys of this block below Nk
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const uint32_t dst = lds0 + st * STAGE + (wave * LPT + i) * RPI * RB;
      uint32_t ko = koff[i], vo = voff[i];
      if (left < kBK) {
        const int row = (wave * LPT + i) * RPI + lane / CPR;
        const int64_t r = row < left ? row : left - 1;
        ko = (uint32_t)(r * p.ldk * E) + ((pos ^ kswz<CPR>(row)) << 4);
        vo = (uint32_t)(r * p.ldv * E) + ((pos ^ vswz<CPR>(row)) << 4);
      }
      dma16(kbase, ko, dst);
      dma16(vbase, vo, dst + TILE);
    }
  };

  f32x16 acc_o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[b][r] = 0.f;
  // Running maximum m (of c * score, base-2 units) and exp-sum l of this
  // lane's query.  m is raised only when a block's maximum exceeds it by
  // more than kLazy, so weights 2^(c s - m) stay below 2^kLazy and the
  // rescaling of O and l is skipped for most blocks; O / l is the same for
  // any m at or below the true maximum.
  constexpr float kLazy = 8.f;
  float m_run = -__builtin_inff(), l_run = 0.f;

  const int64_t nblk = (Nk + kBK - 1) / kBK;
  const int64_t nfull = Nk / kBK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) lgkmcnt(0)
  __syncthreads();

  auto block = [&](int64_t kb, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const int st = (int)(kb & 1);
    if (kb + 1 < nblk) issue(kb + 1, st ^ 1);
    const char *Kt = lds + st * STAGE;
    const char *Vt = Kt + TILE;

    // ---- S^T = K Q^T for the two 32-key halves of the block
    f32x16 acc_s[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_s[h2][r] = 0.f;
      const int row = 32 * h2 + l32;
#pragma unroll
      for (int c = 0; c < DS; ++c) {
        const i32x4 kf = *(const i32x4 *)(Kt + row * RB + (((2 * c + g) ^ kswz<CPR>(row)) << 4));
        if constexpr (IT == kBF16)
          acc_s[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qf[c]), acc_s[h2], 0, 0, 0);
        else
          acc_s[h2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8, kf), __builtin_bit_cast(f16x8, qf[c]), acc_s[h2], 0, 0, 0);
      }
    }

    // ---- online softmax of this lane's query.  Register r of half h2
    // holds key 32 h2 + 8 (r / 4) + 4 g + r % 4 of the block.
    const int left = kMasked ? (int)(Nk - kb * kBK) : kBK;
    float mloc = -__builtin_inff();
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (kMasked && 32 * h2 + 8 * (r >> 2) + 4 * g + (r & 3) >= left) acc_s[h2][r] = -__builtin_inff();
        mloc = __builtin_fmaxf(mloc, acc_s[h2][r]);
      }
    mloc = __builtin_fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float mcand = mloc * c2;   // finite: each block has a key below Nk
    const bool raise = mcand > m_run + kLazy;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mcand : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[b][r] *= alpha;
    }
    const float nm = -m_run;
    float lsum = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[h2][r], c2, nm));
        if (kMasked && 32 * h2 + 8 * (r >> 2) + 4 * g + (r & 3) >= left) e = 0.f;
        acc_s[h2][r] = e;
        lsum += e;
      }
    lsum += __shfl_xor(lsum, 32, 64);
    l_run += lsum;

    // ---- O^T += V^T P^T, 16 keys per instruction.  Key chunk (h2, h):
    // positions 0-3 of a lane are keys base + 4 g + 0..3 and positions 4-7
    // keys base + 8 + 4 g + 0..3 (base = 32 h2 + 16 h) -- in P^T those are
    // registers 8 h .. 8 h + 7 of half h2; in V^T two transposing reads.
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        i32x4 pf;
#pragma unroll
        for (int w = 0; w < 4; ++w) pf[w] = (int)pack2<IT>(acc_s[h2][8 * h + 2 * w], acc_s[h2][8 * h + 2 * w + 1]);
        const int base = 32 * h2 + 16 * h;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          s16x4 tr[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int row = base + 8 * t + 4 * (G >> 1) + (q16 >> 2);
            const int col = 32 * b + 16 * (G & 1) + 4 * (q16 & 3);   // element column
            const int chunk = col >> 3, within = (col & 7) * E;
            tr[t] = lds_read_tr16(Vt + row * RB + ((chunk ^ vswz<CPR>(row)) << 4) + within);
          }
          const i32x2 t0 = __builtin_bit_cast(i32x2, tr[0]), t1 = __builtin_bit_cast(i32x2, tr[1]);
          const i32x4 vf = {t0[0], t0[1], t1[0], t1[1]};
          if constexpr (IT == kBF16)
            acc_o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, vf), __builtin_bit_cast(bf16x8, pf), acc_o[b], 0, 0, 0);
          else
            acc_o[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, vf), __builtin_bit_cast(f16x8, pf), acc_o[b], 0, 0, 0);
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(0);   // next block's loads and this block's reads done
    __syncthreads();
  };

  for (int64_t kb = 0; kb < nfull; ++kb) block(kb, std::false_type{});
  if (nfull < nblk) block(nfull, std::true_type{});

  // ---- O = O^T / l: lane (query q0 + l32, g), block b, register r holds
  // column 32 b + 8 (r / 4) + 4 g + r % 4; four consecutive columns per store.
  const int64_t q = q0 + l32;
  if (q < Nq) {
    const float inv = 1.f / l_run;
    char *Oq = (char *)p.O + (z * p.strideO + q * p.ldo) * OE;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = 32 * b + 8 * r4 + 4 * g;
        const float v0 = acc_o[b][4 * r4] * inv, v1 = acc_o[b][4 * r4 + 1] * inv;
        const float v2 = acc_o[b][4 * r4 + 2] * inv, v3 = acc_o[b][4 * r4 + 3] * inv;
        if constexpr (OT == kF32) {
          typedef float f32x4 __attribute__((ext_vector_type(4)));
          *(f32x4 *)(Oq + col * 4) = f32x4{v0, v1, v2, v3};
        } else {
          *(i32x2 *)(Oq + col * 2) = i32x2{(int)pack2<OT>(v0, v1), (int)pack2<OT>(v2, v3)};
        }
      }
  }
}

template <int IT, int OT>
hipError_t launch_typed(int D, const AttnParams &p, hipStream_t stream) {
  const int64_t blocks = p.Z * ((p.Nq + kBQ - 1) / kBQ);
  if (D == 128)
    hipLaunchKernelGGL((attn_fwd_kernel<IT, OT, 128>), dim3((unsigned)blocks), dim3(64 * kWaves), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<IT, OT, 64>), dim3((unsigned)blocks), dim3(64 * kWaves), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(Fmt in, Fmt out, int D, const AttnParams &p, hipStream_t stream) {
  if (in == kF16) return out == kF32 ? launch_typed<kF16, kF32>(D, p, stream)
                                     : launch_typed<kF16, kF16>(D, p, stream);
  if (in == kBF16) return out == kF32 ? launch_typed<kBF16, kF32>(D, p, stream)
                                      : launch_typed<kBF16, kBF16>(D, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace tmm
