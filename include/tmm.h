/*
 * tmm.h -- tiled dense matrix multiplication on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libtmm.so.  Three entry points compute
 *
 *     C = scale_a * scale_b * A . op(B)  (+ bias broadcast over rows)
 *
 * for one matrix (tmm_gemm), for a batch of equally shaped matrices at fixed
 * element strides (tmm_gemm_strided_batched), and for the matrix-vector case
 * y = W . x (+ bias) (tmm_gemv).
 *
 * Sources of the operation:
 *   - product definition C[i][j] = sum_k A[i][k] * B[k][j], A (M,K), B (K,N):
 *     "GEMM to FlashAttention" page (youngju.dev), naive_matmul listing;
 *   - the BLAS interface C = alpha*op(A)*op(B) + beta*C with transpose flags,
 *     dimensions m, n, k and leading dimensions lda/ldb/ldc as memory strides:
 *     same page, "GEMM interface" box.  Here only op(B) may be transposed,
 *     alpha is the product of two fp8 dequantisation scales, and beta is 0
 *     (C is overwritten, never read);
 *   - bias as one value per output feature added after the product, weights
 *     stored (out_features, in_features): same page, linear-layer formula;
 *     CMU 15-418 Lecture 27 notes (runguoli.com) section 2.1, fully
 *     connected layer as a matrix-vector product plus b;
 *   - low-precision inputs with fp32 accumulation: Lecture 27 notes section
 *     2.7 (formats, Table 1, "accumulate in higher precision");
 *   - matrix-vector product as the memory-bound Level-2 case: "GEMM to
 *     FlashAttention" page, BLAS levels list; Lecture 27 notes section 7,
 *     question 1 (batch-1 y = W x).
 *
 * Layout: every matrix is row-major.  Element (r, c) of a matrix with
 * leading dimension ld is at element offset r*ld + c from its pointer.
 *   A : M x K, lda >= max(1, K)
 *   B : trans_b == 0 -> K x N, ldb >= max(1, N)       (op(B) = B,   "NN")
 *       trans_b != 0 -> N x K, ldb >= max(1, K)       (op(B) = B^T, "NT";
 *                                                      a linear layer's W)
 *   C : M x N, ldc >= max(1, N)
 *   bias : NULL, or N float32 values (bias[j] is added to column j)
 *
 * Types (ab_type -> allowed c_type):
 *   TMM_F32    -> TMM_F32
 *   TMM_BF16   -> TMM_F32, TMM_BF16
 *   TMM_F16    -> TMM_F32, TMM_F16
 *   TMM_F8E4M3 -> TMM_F32, TMM_BF16        (OCP E4M3, largest finite 448)
 * Products are summed in fp32; a rounded output (bf16/fp16) is rounded once,
 * to nearest even, after scale and bias.  fp16 subnormal inputs and outputs
 * are kept, never flushed.  scale_a and scale_b must be 1 unless ab_type is
 * TMM_F8E4M3; they are the per-tensor dequantisation factors of A and B.
 *
 * Ownership: every pointer is device memory owned by the caller.  The library
 * allocates nothing, keeps no pointer after returning, holds no state between
 * calls and may be called from several host threads at once.  Work is
 * enqueued on `stream` (NULL = the default stream) and the call returns
 * without waiting for it.  C must not overlap A, B or bias.
 *
 * Errors: each call returns TMM_OK (0) or one of the negative codes below.
 * Argument checks run on the host before any HIP call; a failing call
 * enqueues nothing, prints nothing and never exits.  TMM_ERR_LAUNCH reports a
 * HIP error seen right after the launch.
 *
 * Size limits: A and B of one problem must each span less than 4 GiB
 * (the kernels address them with 32-bit byte offsets), and the number of
 * 128 x 128 output tiles times batch must stay below 2^31; otherwise the
 * call returns TMM_ERR_DIM.
 *
 * Quick returns: M == 0, N == 0 or batch == 0 enqueue nothing and return 0
 * (pointers are not checked then).  K == 0 is the empty sum: C = bias (or 0).
 */
#ifndef TMM_H
#define TMM_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tmm_dtype {
  TMM_F32 = 0,
  TMM_BF16 = 1,
  TMM_F16 = 2,
  TMM_F8E4M3 = 3
} tmm_dtype;

enum tmm_status {
  TMM_OK = 0,
  TMM_ERR_DIM = -1,    /* M, N, K or batch negative, or a problem too large  */
  TMM_ERR_LD = -2,     /* a leading dimension below its row length (or < 1)  */
  TMM_ERR_NULL = -3,   /* NULL pointer for an operand with non-zero extent    */
  TMM_ERR_DTYPE = -4,  /* unknown type or a type pair not in the table above  */
  TMM_ERR_SCALE = -5,  /* scale != 1 for a non-fp8 type, or a non-finite one  */
  TMM_ERR_STRIDE = -6, /* negative batch stride, or C matrices that overlap   */
  TMM_ERR_ALIGN = -7,  /* pointer not aligned to its element size            */
  TMM_ERR_LAUNCH = -8, /* HIP reported an error at launch                     */
  TMM_ERR_ARG = -9,    /* unknown activation code or pooling factor, or a    */
                       /* split count outside 1..64 or not dividing K        */
  TMM_ERR_WORKSPACE = -10 /* workspace missing, too small or misaligned      */
};

/* Activation applied last by tmm_gemm_ex. */
typedef enum tmm_activation {
  TMM_ACT_NONE = 0,
  TMM_ACT_RELU = 1 /* max(0, x) */
} tmm_activation;

/*
 * C = scale_a*scale_b * A . op(B) (+ bias).  M x N outputs, K-long sums.
 * A, B, C, bias and the dimensions as described above.
 */
int tmm_gemm(int64_t M, int64_t N, int64_t K, tmm_dtype ab_type,
             tmm_dtype c_type, int trans_b, const void *A, int64_t lda,
             const void *B, int64_t ldb, void *C, int64_t ldc,
             const float *bias, float scale_a, float scale_b,
             hipStream_t stream);

/*
 * The same product for batch = 0, 1, 2, ... independent problems:
 *   C + z*strideC = scale_a*scale_b * (A + z*strideA) . op(B + z*strideB) (+ bias)
 * Strides are in elements and must be >= 0 (0 repeats one operand for every
 * problem).  For batch > 1 the C matrices must not overlap:
 * strideC >= (M-1)*ldc + N.  The one bias vector serves every problem.
 * This is the form of attention's two products, scores = Q . K^T (NT) and
 * output = weights . V (NN), over batch x heads: "GEMM to FlashAttention"
 * page, attention_standard listing.
 */
int tmm_gemm_strided_batched(int64_t M, int64_t N, int64_t K,
                             tmm_dtype ab_type, tmm_dtype c_type, int trans_b,
                             const void *A, int64_t lda, int64_t strideA,
                             const void *B, int64_t ldb, int64_t strideB,
                             void *C, int64_t ldc, int64_t strideC,
                             int64_t batch, const float *bias, float scale_a,
                             float scale_b, hipStream_t stream);

/*
 * y[n] = sum_k W[n][k] * x[k] (+ bias[n]),  n < N, k < K.
 *   W : N x K row-major (out_features x in_features), ldw >= max(1, K)
 *   x : K elements of w_type;  y : N elements of y_type
 * w_type -> y_type as for tmm_gemm, except that TMM_F8E4M3 is not accepted.
 * A memory-bound stream over W: every weight is read once.
 */
int tmm_gemv(int64_t N, int64_t K, tmm_dtype w_type, tmm_dtype y_type,
             const void *W, int64_t ldw, const void *x, void *y,
             const float *bias, hipStream_t stream);

/*
 * Fused attention forward, one head per batch entry z < batch:
 *   O[z][i][c] = sum_j w[i][j] V[z][j][c],
 *   w[i][j] = exp(s[i][j]) / sum_j' exp(s[i][j']),   s = scale * Q[z] . K[z]^T
 * ("GEMM to FlashAttention" page: the attention formula and the
 * attention_standard listing, whose scale defaults to 1/sqrt(D); evaluated
 * with the online softmax of its flash_attention_simplified listing, so the
 * Nq x Nk scores never reach memory).  No mask.
 *   Q : Nq x D rows at ldq, K and V : Nk x D rows at ldk / ldv, O : Nq x D
 *   rows at ldo; batch strides in elements, >= 0 (the O matrices must not
 *   overlap: strideO >= (Nq-1)*ldo + D when batch > 1).
 *   in_type: TMM_F16 or TMM_BF16 (Q, K, V alike); out_type: in_type or
 *   TMM_F32.  Scores and sums are fp32; the weights enter the second product
 *   rounded to in_type.
 *   D must be 64 or 128 (TMM_ERR_DIM otherwise); Nk >= 1 when Nq > 0
 *   (TMM_ERR_DIM); every pointer 16-byte aligned and every ld and stride a
 *   multiple of 8 elements (TMM_ERR_ALIGN); ldk, ldv <= 2^24 (TMM_ERR_LD);
 *   scale finite, also times log2(e) (TMM_ERR_SCALE).
 * Quick return: batch == 0 or Nq == 0.
 */
int tmm_attention_fwd(int64_t batch, int64_t Nq, int64_t Nk, int64_t D,
                      tmm_dtype in_type, tmm_dtype out_type,
                      const void *Q, int64_t ldq, int64_t strideQ,
                      const void *K, int64_t ldk, int64_t strideK,
                      const void *V, int64_t ldv, int64_t strideV,
                      void *O, int64_t ldo, int64_t strideO, float scale,
                      hipStream_t stream);

/*
 * The full BLAS form with a fused activation, batched:
 *   C[z] = act( alpha * op(A[z]) . op(B[z]) + bias + beta * C[z] )
 * with op(A) = A (M x K, lda >= K) or A^T (A stored K x M, lda >= M) by
 * trans_a, op(B) = B (K x N, ldb >= N) or B^T (B stored N x K, ldb >= K) by
 * trans_b, for z < batch at strides strideA / strideB / strideC (elements).
 * ("GEMM to FlashAttention" page: the BLAS level-3 gemm and the GEMM
 * interface box, transa / transb / alpha / beta / lda / ldb / ldc; CMU
 * 15-418 Lecture 27 notes section 2.1: a unit computes f(sum x w + b) with
 * f = ReLU, and the fused scale / bias / ReLU epilogue of section 3.1.)
 *   The sum is fp32; alpha * sum + bias + beta * old C is formed in fp32,
 *   the activation applied (TMM_ACT_NONE or TMM_ACT_RELU, else TMM_ERR_ARG)
 *   and the result rounded once (nearest even) to c_type.  beta == 0 does
 *   not read C (it may hold anything); alpha and beta must be finite
 *   (TMM_ERR_SCALE).  For fp8 inputs alpha carries the dequantisation
 *   scales.  Type pairs as for tmm_gemm; trans_a needs bf16 or fp16 inputs
 *   (TMM_ERR_DTYPE otherwise).  Quick returns as for tmm_gemm; K == 0 gives
 *   C = act(bias + beta * old C).  Other limits and errors as for
 *   tmm_gemm_strided_batched.
 */
int tmm_gemm_ex(int64_t M, int64_t N, int64_t K, tmm_dtype ab_type, tmm_dtype c_type,
                int trans_a, int trans_b, const void *A, int64_t lda, int64_t strideA,
                const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                int64_t strideC, int64_t batch, const float *bias, float alpha, float beta,
                int activation, hipStream_t stream);

/*
 * Fused stride-1 2-D convolution, NHWC, as an implicit GEMM:
 *   out[n][oy][ox][f] = pool over the 2 x 2 block of (y, x) (pool == 2) or
 *   (y, x) = (oy, ox) (pool == 1) of
 *     act( scale[f] * sum_{r,s,c} w[f][r][s][c] in[n][y+r-pad][x+s-pad][c] + bias[f] )
 * with inputs outside the H x W image taken as 0.  (CMU 15-418 Lecture 27
 * notes: the convolution loop nest of section 2.2, implicit GEMM in section
 * 2.3, and the conv_fused listing of section 3.1 -- NHWC input with a zero
 * halo, weights [K][R][S][C], per-filter scale and bias, ReLU, 2 x 2 max
 * pooling.)
 *   in : N x H x W x C, contiguous; w : K x R x S x C, contiguous; out :
 *   N x OH x OW x K, contiguous, OH = (H + 2 pad - R + 1) / pool, OW alike.
 *   scale, bias: K floats each or NULL (1 and 0).  in_type TMM_BF16 or
 *   TMM_F16 (in and w alike), out_type in_type or TMM_F32; sums in fp32, one
 *   nearest-even rounding after the pooling.
 *   Limits: C a multiple of 8 and in, w 16-byte aligned (TMM_ERR_ALIGN);
 *   N >= 0, H, W, C, K, R, S >= 1, pad >= 0, output size >= 1 and even
 *   when pool == 2, R*S*C and every dimension below 2^31 (TMM_ERR_DIM);
 *   pool 1 or 2 and activation TMM_ACT_NONE / TMM_ACT_RELU (TMM_ERR_ARG).
 *   Quick return for N == 0.
 */
int tmm_conv2d_fused(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                     int64_t pad, tmm_dtype in_type, tmm_dtype out_type, const void *in,
                     const void *w, const float *scale, const float *bias, int activation,
                     int pool, void *out, hipStream_t stream);

/*
 * The product of tmm_gemm with K cut into `splits` equal slices, for
 * products with few rows (the decode end of the batch-size table on the
 * "GEMM to FlashAttention" page, where a one-pass tiling gives every CU its
 * own long stretch of both operands): slice s's fp32 partial product goes to
 * the caller's workspace, then the slices are summed and finished:
 *
 *   W[s] = A[:, s*K/S .. (s+1)*K/S) . op(B)[s*K/S .. (s+1)*K/S, :]   (fp32)
 *   C    = round( scale_a*scale_b * (W[0] + W[1] + ... + W[S-1]) + bias )
 *
 * (S = splits), summed in that fixed order with one nearest-even rounding:
 * the result is deterministic and within the fp32 summation bound of the
 * one-pass product (the bias and scale as in tmm_gemm, the GEMM page's
 * linear-layer formula and interface box).
 *   splits    : 1 .. 64 dividing K (TMM_ERR_ARG); splits == 1 or K == 0 is
 *               the one-pass product and leaves the workspace untouched
 *   workspace : device memory of at least splits*M*N*4 bytes, 16-byte
 *               aligned, owned by the caller and overlapping no operand
 *               (TMM_ERR_WORKSPACE when NULL, smaller or misaligned); its
 *               contents on return are unspecified.  Calls that share one
 *               workspace must be ordered (same stream, or synchronised).
 * Every other argument, type pair, limit and error as for tmm_gemm.
 */
int tmm_gemm_splitk(int64_t M, int64_t N, int64_t K, tmm_dtype ab_type, tmm_dtype c_type,
                    int trans_b, const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                    int64_t ldc, const float *bias, float scale_a, float scale_b, int splits,
                    void *workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * tmm_gemm_splitk without the workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The partial products go to a scratch
 * array the library holds on each GPU it runs on, TMM_SPLITK_SCRATCH_BYTES
 * (32 MiB) per GPU, kept until the process ends; this call allocates
 * nothing.  A problem needing more than that (splits*M*N*4 bytes) returns
 * TMM_ERR_WORKSPACE before any HIP call.  Every call on one GPU shares that
 * GPU's scratch: calls that overlap on a GPU (on concurrent streams or host
 * threads) race and must be ordered by the caller.  Everything else as for
 * tmm_gemm_splitk.
 */
#define TMM_SPLITK_SCRATCH_BYTES 33554432
int tmm_gemm_splitk_noalloc(int64_t M, int64_t N, int64_t K, tmm_dtype ab_type, tmm_dtype c_type,
                            int trans_b, const void *A, int64_t lda, const void *B, int64_t ldb,
                            void *C, int64_t ldc, const float *bias, float scale_a, float scale_b,
                            int splits, hipStream_t stream);

/* Static English text of a status code (never NULL). */
const char *tmm_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int tmm_version(void);

/*
 * Kernel-choice override, for measurements and kernel-by-kernel tests only;
 * results are the same (within the stated tolerances) whatever it pins.
 * `spec` is a list of key=value items separated by ';' or spaces, NULL or ""
 * for none:
 *   tile=256x256 | 256x128 | 128x128 | 256x256w4 | 256x256s2 | 256x256r |
 *        256x256q | 256x128q | 128x128q | skinny | generic | shortk | gemvm
 *                  the GEMM kernel / tile shape wherever it applies
 *                  (256x256s2: two-stage kernel only; 256x256r: the ring
 *                  kernel, K-contiguous B included; ...q: the four-wave
 *                  kernel with 16x16x32 instructions; skinny, generic, shortk,
 *                  gemvm: the skinny-M, any-layout, short-K and several-row
 *                  GEMV kernels)
 *   skinny=<bm>x<bn>   skinny-M tile, bm and bn in {16, 32, 64}
 *   gemv=<r>x<w>       GEMV rows per wave (1, 2, 4) and waves per workgroup
 *                      (4, 8, 16)
 *   conv=quad | direct the convolution kernel: LDS-staged 128-pixel x
 *                      128-filter tiles (taken only where C % 32 == 0 and
 *                      R S C >= 96) or register-direct 128/256 x 64 tiles
 *   ring=4 | 8         stages of the four-wave kernel's ring on 128x128
 *                      tiles (8: plain epilogue and at least 8 ring steps
 *                      only; chosen by the grid's size otherwise)
 * The same text in the environment variable TMM_OVERRIDE is read once, at
 * the library's first call (an unparsable value pins nothing).  This call
 * replaces the whole setting for every later call from any thread; calls
 * already enqueued keep their kernels.  Returns TMM_OK, or TMM_ERR_ARG for
 * an unknown key or value (the setting is then left as it was).
 */
int tmm_set_override(const char *spec);

#ifdef __cplusplus
}
#endif

#endif /* TMM_H */
