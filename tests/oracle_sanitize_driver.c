/* Runs every oracle entry point once per format and layout on small
 * problems whose buffers are allocated to their exact extents (last row
 * without padding), so that a build with -fsanitize=address,undefined
 * (tests/test_oracle_sanitize.py) reports any access outside them or any
 * undefined behaviour.  Also checks a few results that are known exactly. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_decode(int fmt, const void *src, double *dst, int64_t n);
int oracle_round(int fmt, const double *src, uint16_t *dst, int64_t n);
int oracle_gemm(int64_t M, int64_t N, int64_t K, int fmt, const void *A, int64_t lda, const void *B,
                int64_t ldb, int trans_b, const float *bias, double scale_a, double scale_b, double *C,
                int64_t ldc, double *T);
int oracle_gemm_ex(int64_t M, int64_t N, int64_t K, int fmt, int trans_a, int trans_b, const void *A,
                   int64_t lda, const void *B, int64_t ldb, double alpha, double beta, const double *Cin,
                   const float *bias, int act, double *C, int64_t ldc, double *T);
int oracle_attention(int64_t Nq, int64_t Nk, int64_t D, int fmt, const void *Q, int64_t ldq, const void *K,
                     int64_t ldk, const void *V, int64_t ldv, double scale, double *O, int64_t ldo, double *T);
int oracle_conv2d(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S, int64_t pad,
                  int fmt, const void *in, const void *w, const float *scale, const float *bias, int relu,
                  int pool, double *out, double *T);

static const int esz[4] = {4, 2, 2, 1};
/* bit patterns of 1.0 per format: f32, bf16, f16, e4m3 */
static const uint32_t one_bits[4] = {0x3f800000u, 0x3f80u, 0x3c00u, 0x38u};

static void *ones(int fmt, int64_t n) {
  void *p = malloc((size_t)(n > 0 ? n : 1) * esz[fmt]);
  for (int64_t i = 0; i < n; ++i) {
    if (esz[fmt] == 4) ((uint32_t *)p)[i] = one_bits[fmt];
    else if (esz[fmt] == 2) ((uint16_t *)p)[i] = (uint16_t)one_bits[fmt];
    else ((uint8_t *)p)[i] = (uint8_t)one_bits[fmt];
  }
  return p;
}

static int fails = 0;
#define EXPECT(c, ...) do { if (!(c)) { printf("FAIL: " __VA_ARGS__); printf("\n"); ++fails; } } while (0)

int main(void) {
  for (int fmt = 0; fmt < 4; ++fmt) {
    /* decode / round */
    {
      const int64_t n = 37;
      void *src = ones(fmt, n);
      double *d = malloc(n * sizeof(double));
      EXPECT(oracle_decode(fmt, src, d, n) == 0, "decode fmt %d", fmt);
      for (int64_t i = 0; i < n; ++i) EXPECT(d[i] == 1.0, "decode value fmt %d", fmt);
      if (fmt == 1 || fmt == 2) {
        uint16_t *r = malloc(n * sizeof(uint16_t));
        EXPECT(oracle_round(fmt, d, r, n) == 0, "round fmt %d", fmt);
        for (int64_t i = 0; i < n; ++i) EXPECT(r[i] == (uint16_t)one_bits[fmt], "round value fmt %d", fmt);
        free(r);
      }
      free(src);
      free(d);
    }
    /* plain and full-form products, every layout, padded leading dimensions */
    for (int ta = 0; ta <= 1; ++ta)
      for (int tb = 0; tb <= 1; ++tb) {
        const int64_t M = 5, N = 7, K = 9;
        const int64_t lda = (ta ? M : K) + 3, ldb = (tb ? K : N) + 2, ldc = N + 1;
        const int64_t nA = (ta ? (K - 1) * lda + M : (M - 1) * lda + K);
        const int64_t nB = (tb ? (N - 1) * ldb + K : (K - 1) * ldb + N);
        const int64_t nC = (M - 1) * ldc + N;
        void *A = ones(fmt, nA), *B = ones(fmt, nB);
        float *bias = malloc(N * sizeof(float));
        double *Cin = malloc(nC * sizeof(double)), *C = malloc(nC * sizeof(double)),
               *T = malloc(nC * sizeof(double));
        for (int64_t j = 0; j < N; ++j) bias[j] = (float)j;
        for (int64_t i = 0; i < nC; ++i) Cin[i] = 1.0;
        if (!ta) {
          EXPECT(oracle_gemm(M, N, K, fmt, A, lda, B, ldb, tb, bias, 1.0, 1.0, C, ldc, T) == 0, "gemm");
          for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j)
              EXPECT(C[i * ldc + j] == K + j && T[i * ldc + j] == K, "gemm value fmt %d", fmt);
        }
        EXPECT(oracle_gemm_ex(M, N, K, fmt, ta, tb, A, lda, B, ldb, 2.0, -1.0, Cin, bias, 1, C, ldc, T) == 0,
               "gemm_ex");
        for (int64_t i = 0; i < M; ++i)
          for (int64_t j = 0; j < N; ++j)
            EXPECT(C[i * ldc + j] == 2.0 * K + j - 1.0 && T[i * ldc + j] == 2.0 * K + j + 1.0,
                   "gemm_ex value fmt %d", fmt);
        free(A); free(B); free(bias); free(Cin); free(C); free(T);
      }
    /* attention of one head: all-ones inputs give o = 1 */
    {
      const int64_t Nq = 3, Nk = 5, D = 4, ldq = D + 1, ldk = D + 2, ldv = D + 3, ldo = D + 1;
      void *Q = ones(fmt, (Nq - 1) * ldq + D), *Kt = ones(fmt, (Nk - 1) * ldk + D),
           *V = ones(fmt, (Nk - 1) * ldv + D);
      double *O = malloc(((Nq - 1) * ldo + D) * sizeof(double)), *T = malloc(((Nq - 1) * ldo + D) * sizeof(double));
      EXPECT(oracle_attention(Nq, Nk, D, fmt, Q, ldq, Kt, ldk, V, ldv, 0.5, O, ldo, T) == 0, "attention");
      for (int64_t i = 0; i < Nq; ++i)
        for (int64_t c = 0; c < D; ++c) EXPECT(O[i * ldo + c] == 1.0, "attention value fmt %d", fmt);
      free(Q); free(Kt); free(V); free(O); free(T);
    }
    /* convolution, pooled and not */
    for (int pool = 1; pool <= 2; ++pool) {
      const int64_t N = 2, H = 4, W = 6, C = 3, K = 2, R = 3, S = 3, pad = 1;
      const int64_t OH = (H + 2 * pad - R + 1) / pool, OW = (W + 2 * pad - S + 1) / pool;
      void *in = ones(fmt, N * H * W * C), *w = ones(fmt, K * R * S * C);
      float scale[2] = {1.0f, 2.0f}, bias[2] = {0.5f, -0.5f};
      double *out = malloc(N * OH * OW * K * sizeof(double)), *T = malloc(N * OH * OW * K * sizeof(double));
      EXPECT(oracle_conv2d(N, H, W, C, K, R, S, pad, fmt, in, w, scale, bias, 1, pool, out, T) == 0, "conv");
      /* an interior pixel sees all 27 taps */
      if (pool == 1) EXPECT(out[((0 * OH + 1) * OW + 1) * K + 1] == 2.0 * 27 - 0.5, "conv value fmt %d", fmt);
      free(in); free(w); free(out); free(T);
    }
  }
  if (fails) {
    printf("%d failures\n", fails);
    return 1;
  }
  printf("OK\n");
  return 0;
}
