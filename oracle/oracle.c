/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU statement of what the GPU library
 * computes.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load this file's library.  It shares no code, header, table
 * or helper with the HIP library; it never calls it and is never called by it.
 *
 * What it computes (all in IEEE double precision):
 *
 *   o[i][j] = s_a * s_b * sum_{k<K} a[i][k] * b'[k][j]  (+ bias[j])
 *
 *   - the definition C[i][j] = sum_k A[i][k]*B[k][j] with a float64
 *     accumulator: "GEMM to FlashAttention" page (youngju.dev), the
 *     naive_matmul listing;
 *   - op(B) = B or B^T selected by a transpose flag, leading dimensions as
 *     memory strides: same page, the BLAS "GEMM interface" box;
 *   - the bias is one value per output feature, added after the product:
 *     same page, the linear-layer formula at its top, and CMU 15-418
 *     Lecture 27 notes (runguoli.com) section 2.1 (fully connected layer =
 *     matrix-vector product plus b);
 *   - inputs are stored in a low-precision format and the products are summed
 *     at higher precision: Lecture 27 notes section 2.7 (formats figure and
 *     Table 1).  Here the sum is exact-ish fp64 over the exactly decoded
 *     inputs, which is the plain definition the fp32-accumulating kernels
 *     approximate.
 *
 * Input formats are decoded exactly from their bit patterns by the decoders
 * below, each written from the format's definition (Lecture 27 notes
 * section 2.7 gives the bit splits: fp32 1+8+23, bf16 1+8+7, fp8 E4M3 1+4+3
 * with range to 448; fp16 is IEEE binary16, 1+5+10).
 *
 * Output rounding R(o) to bf16 / fp16 is "round to the nearest representable
 * value, ties to the even significand", written from that definition on the
 * format's grid of representable values.
 *
 * oracle_gemm_ex states the full BLAS form the same way (see there).
 *
 * oracle_attention states softmax(scale Q K^T) V the same way (see there),
 * and oracle_conv2d the fused convolution (see there).
 *
 * Each pin of this file lives in tests/test_oracle.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The oracle's own format codes (its own numbering). */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F16 2
#define ORC_E4M3 3

/* ---------------- decoders: bit pattern -> exact double ---------------- */

static double dec_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* bf16 is the upper half of an fp32 pattern: same sign and exponent field,
 * the top 7 of the 23 fraction bits. */
static double dec_bf16(uint16_t u) { return dec_f32((uint32_t)u << 16); }

/* IEEE binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static double dec_f16(uint16_t u) {
  int s = (u >> 15) & 1;
  int e = (u >> 10) & 0x1f;
  int m = u & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + m, e - 25); /* (1 + m/2^10) * 2^(e-15) */
  return s ? -v : v;
}

/* OCP fp8 E4M3 ("fn"): sign, 4-bit exponent (bias 7), 3-bit fraction, no
 * infinities, S.1111.111 is NaN, largest finite 1.75 * 2^8 = 448. */
static double dec_e4m3(uint8_t u) {
  int s = (u >> 7) & 1;
  int e = (u >> 3) & 0xf;
  int m = u & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9); /* m/8 * 2^-6 */
  else
    v = ldexp(8.0 + m, e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

static double dec_at(int fmt, const void *p, int64_t idx) {
  switch (fmt) {
  case ORC_F32:
    return dec_f32(((const uint32_t *)p)[idx]);
  case ORC_BF16:
    return dec_bf16(((const uint16_t *)p)[idx]);
  case ORC_F16:
    return dec_f16(((const uint16_t *)p)[idx]);
  case ORC_E4M3:
    return dec_e4m3(((const uint8_t *)p)[idx]);
  default:
    return NAN;
  }
}

int oracle_decode(int fmt, const void *src, double *dst, int64_t n) {
  if (fmt < ORC_F32 || fmt > ORC_E4M3 || n < 0)
    return -1;
  for (int64_t i = 0; i < n; ++i)
    dst[i] = dec_at(fmt, src, i);
  return 0;
}

/* ---------------- rounding: double -> nearest format value ---------------- */

/*
 * Round x to the grid of a binary format with `p` significant bits and
 * smallest normal exponent `emin` (values are (1.f) * 2^e, e >= emin, and
 * subnormals share the grid spacing 2^(emin-p+1)).  Ties go to the value
 * whose last significand bit is zero: rint() in the default rounding mode
 * does exactly that on the integer grid x / quantum.
 */
static double round_to_grid(double x, int p, int emin) {
  if (x == 0.0 || !isfinite(x))
    return x;
  int ex;
  frexp(fabs(x), &ex); /* |x| = f * 2^ex, f in [0.5, 1): exponent e = ex-1 */
  int e = ex - 1;
  if (e < emin)
    e = emin;
  double quantum = ldexp(1.0, e - (p - 1));
  return rint(x / quantum) * quantum; /* x/quantum and the product are exact */
}

/* bf16: 8 significant bits, emin = -126, largest finite (2 - 2^-7) * 2^127. */
static uint16_t enc_bf16(double x) {
  if (isnan(x))
    return 0x7fc0;
  double r = round_to_grid(x, 8, -126);
  /* r is exactly representable in bf16 unless it overflowed past the top
   * binade, in which case it rounded up to 2^128: infinity. */
  if (fabs(r) >= ldexp(1.0, 128))
    return signbit(x) ? 0xff80 : 0x7f80;
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* fp16: 11 significant bits, emin = -14, largest finite 65504. */
static uint16_t enc_f16(double x) {
  if (isnan(x))
    return 0x7e00;
  double r = round_to_grid(x, 11, -14);
  uint16_t s = signbit(x) ? 0x8000 : 0;
  double a = fabs(r);
  if (a >= 65536.0)
    return s | 0x7c00;
  if (a == 0.0)
    return s;
  if (a < ldexp(1.0, -14)) /* subnormal: a = m * 2^-24 */
    return s | (uint16_t)(a * ldexp(1.0, 24));
  int ex;
  double f = frexp(a, &ex);         /* a = f * 2^ex, f in [0.5,1) */
  int e = ex - 1;                   /* a = (2f) * 2^e, 2f in [1,2) */
  double frac = (2.0 * f - 1.0) * 1024.0; /* exact integer 0..1023 */
  return s | (uint16_t)((e + 15) << 10) | (uint16_t)frac;
}

int oracle_round(int fmt, const double *src, uint16_t *dst, int64_t n) {
  if (n < 0)
    return -1;
  if (fmt == ORC_BF16) {
    for (int64_t i = 0; i < n; ++i)
      dst[i] = enc_bf16(src[i]);
    return 0;
  }
  if (fmt == ORC_F16) {
    for (int64_t i = 0; i < n; ++i)
      dst[i] = enc_f16(src[i]);
    return 0;
  }
  return -1;
}

/* ---------------- the product ---------------- */

/*
 * o = s_a*s_b * A . op(B) (+ bias), everything decoded to double first.
 *
 *   A  : M rows of K elements, row i starts at element i*lda
 *   B  : trans_b == 0 -> K rows of N elements (row k at k*ldb), b'[k][j] = B[k][j]
 *        trans_b != 0 -> N rows of K elements (row j at j*ldb), b'[k][j] = B[j][k]
 *   bias: NULL or N float32 values, added to every row
 *   C  : M rows of N doubles at stride ldc (written, not accumulated into)
 *   T  : NULL or M rows of N doubles at stride ldc, T[i][j] = sum_k |a_ik b'_kj|
 *        (the scale of the rounding error bound of any summation order)
 *
 * Loop order i, k, j with a double row accumulator.  Rows are independent,
 * so they are spread over OpenMP threads; each row's sum is formed the same
 * way whatever the thread count.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K, int fmt, const void *A,
                int64_t lda, const void *B, int64_t ldb, int trans_b,
                const float *bias, double scale_a, double scale_b, double *C,
                int64_t ldc, double *T) {
  if (M < 0 || N < 0 || K < 0 || fmt < ORC_F32 || fmt > ORC_E4M3)
    return -1;
  if (lda < K || ldc < N || ldb < (trans_b ? K : N))
    return -2;
  if (M == 0 || N == 0)
    return 0;

  /* b' as a K x N double matrix (row k contiguous). */
  double *bp = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)N);
  if (!bp)
    return -3;
  for (int64_t k = 0; k < K; ++k)
    for (int64_t j = 0; j < N; ++j)
      bp[k * N + j] = trans_b ? dec_at(fmt, B, j * ldb + k) : dec_at(fmt, B, k * ldb + j);

  const double scale = scale_a * scale_b; /* exact: two floats' product fits a double */
  int fail = 0;

#pragma omp parallel
  {
    double *acc = (double *)malloc(sizeof(double) * (size_t)N);
    double *tab = T ? (double *)malloc(sizeof(double) * (size_t)N) : NULL;
    if (!acc || (T && !tab)) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
          acc[j] = 0.0;
          if (tab)
            tab[j] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
          const double a = dec_at(fmt, A, i * lda + k);
          const double *brow = bp + k * N;
          for (int64_t j = 0; j < N; ++j)
            acc[j] += a * brow[j];
          if (tab)
            for (int64_t j = 0; j < N; ++j)
              tab[j] += fabs(a * brow[j]);
        }
        for (int64_t j = 0; j < N; ++j) {
          double v = scale * acc[j];
          if (bias)
            v += (double)bias[j];
          C[i * ldc + j] = v;
          if (tab)
            T[i * ldc + j] = fabs(scale) * tab[j];
        }
      }
    }
    free(acc);
    free(tab);
  }
  free(bp);
  return fail ? -3 : 0;
}

/*
 * The full BLAS form of the product with a fused activation:
 *
 *   o[i][j] = act( alpha * sum_{k<K} a'[i][k] * b'[k][j] + bias[j] + beta * c[i][j] )
 *
 *   - C = alpha * op(A) * op(B) + beta * C with op = identity or transpose
 *     per operand: "GEMM to FlashAttention" page, the BLAS level-3 line and
 *     the "GEMM interface" box (transa / transb, alpha, beta);
 *   - bias per output feature added to the product, then the activation
 *     f(x) = max(0, x) (ReLU): CMU 15-418 Lecture 27 notes section 2.1 (a
 *     unit computes f(sum_i x_i w_i + b), ReLU one such f) and the fused
 *     scale / bias / ReLU epilogue of its conv_fused listing (section 3.1).
 *     The order bias-then-beta is immaterial in exact arithmetic; the
 *     activation comes last.
 *
 *   A  : trans_a ? K x M : M x K inputs at stride lda  (a' = op(A), M x K)
 *   B  : trans_b ? N x K : K x N inputs at stride ldb  (b' = op(B), K x N)
 *   Cin: NULL (beta ignored) or M x N doubles at stride ldc, the old C
 *   C  : M x N doubles at stride ldc (written; may be the same array as Cin)
 *   T  : NULL or like C: |alpha| sum_k |a' b'| + |bias| + |beta c|, the
 *        scale of the error of any fp32 evaluation
 *   act: 0 none, 1 ReLU
 */
int oracle_gemm_ex(int64_t M, int64_t N, int64_t K, int fmt, int trans_a, int trans_b,
                   const void *A, int64_t lda, const void *B, int64_t ldb, double alpha,
                   double beta, const double *Cin, const float *bias, int act, double *C,
                   int64_t ldc, double *T) {
  if (M < 0 || N < 0 || K < 0 || fmt < ORC_F32 || fmt > ORC_E4M3 || act < 0 || act > 1)
    return -1;
  if (lda < (trans_a ? M : K) || ldb < (trans_b ? K : N) || ldc < N)
    return -2;
  if (M == 0 || N == 0)
    return 0;
  /* a' (M x K) and b' (K x N) as doubles */
  const int64_t Kd = K > 0 ? K : 1;
  double *ap = (double *)malloc(sizeof(double) * (size_t)M * (size_t)Kd);
  double *bp = (double *)malloc(sizeof(double) * (size_t)Kd * (size_t)N);
  if (!ap || !bp) {
    free(ap);
    free(bp);
    return -3;
  }
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k)
      ap[i * Kd + k] = trans_a ? dec_at(fmt, A, k * lda + i) : dec_at(fmt, A, i * lda + k);
  for (int64_t k = 0; k < K; ++k)
    for (int64_t j = 0; j < N; ++j)
      bp[k * N + j] = trans_b ? dec_at(fmt, B, j * ldb + k) : dec_at(fmt, B, k * ldb + j);

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double sum = 0.0, sabs = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double t = ap[i * Kd + k] * bp[k * N + j];
        sum += t;
        sabs += fabs(t);
      }
      const double b = bias ? (double)bias[j] : 0.0;
      const double c = Cin ? beta * Cin[i * ldc + j] : 0.0;
      double v = alpha * sum + b + c;
      if (act == 1 && !(v > 0.0))
        v = 0.0;
      if (T)
        T[i * ldc + j] = fabs(alpha) * sabs + fabs(b) + fabs(c);
      C[i * ldc + j] = v;
    }
  }
  free(ap);
  free(bp);
  return 0;
}

/*
 * Scaled dot-product attention of one head, in double precision:
 *
 *   s[i][j] = scale * sum_{c<D} q[i][c] * k[j][c]
 *   w[i][j] = exp(s[i][j]) / sum_{j'<Nk} exp(s[i][j'])   (softmax over keys)
 *   o[i][c] = sum_{j<Nk} w[i][j] * v[j][c]
 *
 * "GEMM to FlashAttention" page (youngju.dev): the attention formula at its
 * top and the attention_standard listing (scores Q K^T times a scale that
 * defaults to 1/sqrt(d), softmax over the last axis, then times V).  The
 * exponentials are taken of s - max_j s, the same quotient written so that
 * exp cannot overflow.
 *
 *   Q  : Nq rows of D inputs (format fmt) at stride ldq
 *   K  : Nk rows of D inputs at stride ldk
 *   V  : Nk rows of D inputs at stride ldv
 *   O  : Nq rows of D doubles at stride ldo (written)
 *   T  : NULL or like O, T[i][c] = sum_j w[i][j] |v[j][c]| (the scale of
 *        the error of any evaluation that rounds the weights)
 *
 * Rows are independent and spread over OpenMP threads.
 */
int oracle_attention(int64_t Nq, int64_t Nk, int64_t D, int fmt, const void *Q,
                     int64_t ldq, const void *K, int64_t ldk, const void *V,
                     int64_t ldv, double scale, double *O, int64_t ldo, double *T) {
  if (Nq < 0 || Nk < 1 || D < 1 || fmt < ORC_F32 || fmt > ORC_E4M3)
    return -1;
  if (ldq < D || ldk < D || ldv < D || ldo < D)
    return -2;
  int fail = 0;
#pragma omp parallel
  {
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *s = (double *)malloc(sizeof(double) * (size_t)Nk);
    if (!q || !s) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < Nq; ++i) {
        for (int64_t c = 0; c < D; ++c)
          q[c] = dec_at(fmt, Q, i * ldq + c);
        double smax = -HUGE_VAL;
        for (int64_t j = 0; j < Nk; ++j) {
          double dot = 0.0;
          for (int64_t c = 0; c < D; ++c)
            dot += q[c] * dec_at(fmt, K, j * ldk + c);
          s[j] = scale * dot;
          if (s[j] > smax)
            smax = s[j];
        }
        double den = 0.0;
        for (int64_t j = 0; j < Nk; ++j) {
          s[j] = exp(s[j] - smax); /* s now holds the unnormalised weights */
          den += s[j];
        }
        for (int64_t c = 0; c < D; ++c) {
          double acc = 0.0, tab = 0.0;
          for (int64_t j = 0; j < Nk; ++j) {
            const double v = dec_at(fmt, V, j * ldv + c);
            acc += s[j] * v;
            tab += s[j] * fabs(v);
          }
          O[i * ldo + c] = acc / den;
          if (T)
            T[i * ldo + c] = tab / den;
        }
      }
    }
    free(q);
    free(s);
  }
  return fail ? -3 : 0;
}

/* Number of threads the product above runs on. */

/*
 * Direct 2-D convolution with the fused epilogue, stride 1:
 *
 *   conv[n][y][x][f] = sum_{r<R, s<S, c<C} w[f][r][s][c] * in[n][y+r-pad][x+s-pad][c]
 *                      (inputs outside the H x W image are 0)
 *   v = act(conv * scale[f] + bias[f]);  out = v, or the max of v over each
 *   2 x 2 block (y, x) in {2Y, 2Y+1} x {2X, 2X+1} when pool == 2
 *
 * CMU 15-418 Lecture 27 notes: the convolution as the seven-loop nest of
 * section 2.2 and the conv_fused listing of section 3.1 (NHWC input with a
 * zero halo of `pad`, weights [K][R][S][C], per-filter scale and bias,
 * ReLU, 2 x 2 max pooling), in the listing's loop order over (dy, dx, r, s,
 * c) for each pooled output.  The implicit-GEMM view (section 2.3) is not
 * used here: this is the definition.
 *
 *   in  : N x H x W x C inputs (format fmt), NHWC, contiguous
 *   w   : K x R x S x C inputs, contiguous
 *   out : N x OH x OW x K doubles, OH = (H + 2 pad - R + 1) / pool (same for W)
 *   T   : NULL or like out: |scale| sum |w in| + |bias| of the output, the
 *         largest over the pooling window (the error of a max is at most
 *         the largest error of its candidates)
 */
int oracle_conv2d(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                  int64_t pad, int fmt, const void *in, const void *w, const float *scale,
                  const float *bias, int relu, int pool, double *out, double *T) {
  if (N < 0 || H < 1 || W < 1 || C < 1 || K < 1 || R < 1 || S < 1 || pad < 0 ||
      fmt < ORC_F32 || fmt > ORC_E4M3 || (pool != 1 && pool != 2))
    return -1;
  const int64_t P = H + 2 * pad - R + 1, Q = W + 2 * pad - S + 1;
  if (P < 1 || Q < 1 || (pool == 2 && (P % 2 || Q % 2)))
    return -2;
  const int64_t OH = P / pool, OW = Q / pool;
  int fail = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t oy = 0; oy < OH; ++oy) {
      for (int64_t ox = 0; ox < OW; ++ox)
        for (int64_t f = 0; f < K; ++f) {
          double best = 0.0, best_t = 0.0;
          int first = 1;
          for (int64_t dy = 0; dy < pool; ++dy)
            for (int64_t dx = 0; dx < pool; ++dx) {
              const int64_t y = oy * pool + dy, x = ox * pool + dx;
              double acc = 0.0, tab = 0.0;
              for (int64_t r = 0; r < R; ++r)
                for (int64_t s = 0; s < S; ++s) {
                  const int64_t iy = y + r - pad, ix = x + s - pad;
                  if (iy < 0 || iy >= H || ix < 0 || ix >= W)
                    continue;
                  for (int64_t c = 0; c < C; ++c) {
                    const double t = dec_at(fmt, w, ((f * R + r) * S + s) * C + c) *
                                     dec_at(fmt, in, ((n * H + iy) * W + ix) * C + c);
                    acc += t;
                    tab += fabs(t);
                  }
                }
              const double sc = scale ? (double)scale[f] : 1.0;
              const double b = bias ? (double)bias[f] : 0.0;
              double v = acc * sc + b;
              if (relu && !(v > 0.0))
                v = 0.0;
              if (first || v > best)
                best = v;
              const double tv = fabs(sc) * tab + fabs(b);
              if (first || tv > best_t)
                best_t = tv;
              first = 0;
            }
          out[((n * OH + oy) * OW + ox) * K + f] = best;
          if (T)
            T[((n * OH + oy) * OW + ox) * K + f] = best_t;
        }
    }
  return fail ? -3 : 0;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the loops above from now on (timing only; results do not
 * depend on it: every output is summed by one thread in a fixed order). */
int oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0)
    omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}
