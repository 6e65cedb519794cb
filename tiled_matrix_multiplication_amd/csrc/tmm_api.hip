// C-ABI entry points of libtmm.so: argument checks, quick returns, and the
// choice of kernel by shape, type and alignment.  Declarations and the full
// contract are in include/tmm.h.
//
// Every check runs on the host before any HIP call, so a rejected call has
// no side effect and the checks are testable on a machine without a GPU.
#include <stdio.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "tmm.h"
#include "tmm_internal.h"

namespace tmm {

// Compute units of the current device (cached per device; callers may be on
// several host threads).
int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace tmm

namespace {
uint64_t override_word();
}

namespace tmm {
int gemv_override() {
  const uint64_t ov = override_word();
  return (int)((ov >> 24) & 0xff) * 100 + (int)((ov >> 32) & 0xff);
}
int conv_override() { return (int)((override_word() >> 40) & 3); }
int ring_override() {
  const int r = (int)((override_word() >> 42) & 3);
  return r == 1 ? 4 : r == 2 ? 8 : 0;
}
}  // namespace tmm

namespace {

using tmm::Fmt;

constexpr int kVersion = 10000;  // 1.0.0

int elem_bytes(int t) { return t == TMM_F32 ? 4 : t == TMM_F8E4M3 ? 1 : 2; }

bool known_type(int t) { return t >= TMM_F32 && t <= TMM_F8E4M3; }

// ab -> c pairs the kernels implement.
bool pair_ok(int ab, int c) {
  switch (ab) {
    case TMM_F32: return c == TMM_F32;
    case TMM_BF16: return c == TMM_F32 || c == TMM_BF16;
    case TMM_F16: return c == TMM_F32 || c == TMM_F16;
    case TMM_F8E4M3: return c == TMM_F32 || c == TMM_BF16;
    default: return false;
  }
}

bool aligned(const void *p, int bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

int64_t max1(int64_t v) { return v > 1 ? v : 1; }

// Common checks of tmm_gemm and tmm_gemm_strided_batched.  Returns TMM_OK
// and sets *quick when nothing is to be launched.
// The full form's extra arguments (tmm_gemm_ex); the plain entry points
// use alpha = scale_a * scale_b, beta = 0, no activation, trans_a = 0.
struct Ex {
  bool full = false;
  int trans_a = 0;
  float beta = 0.f;
  int act = 0;
  bool no_skinny = false;   // keep the product on the tiled kernels (split-K partials)
};

int check_gemm(int64_t M, int64_t N, int64_t K, int ab, int c, int trans_b, const void *A,
               int64_t lda, int64_t sA, const void *B, int64_t ldb, int64_t sB, const void *C,
               int64_t ldc, int64_t sC, int64_t batch, const float *bias, float scale_a,
               float scale_b, const Ex &ex, bool *quick) {
  *quick = false;
  if (M < 0 || N < 0 || K < 0 || batch < 0) return TMM_ERR_DIM;
  if (!known_type(ab) || !known_type(c) || !pair_ok(ab, c)) return TMM_ERR_DTYPE;
  if (ex.trans_a && ab != TMM_BF16 && ab != TMM_F16) return TMM_ERR_DTYPE;
  if (!isfinite(scale_a) || !isfinite(scale_b) || !isfinite(scale_a * scale_b) || !isfinite(ex.beta))
    return TMM_ERR_SCALE;
  if (!ex.full && ab != TMM_F8E4M3 && (scale_a != 1.0f || scale_b != 1.0f)) return TMM_ERR_SCALE;
  if (ex.act != 0 && ex.act != 1) return TMM_ERR_ARG;
  if (lda < max1(ex.trans_a ? M : K) || ldb < max1(trans_b ? K : N) || ldc < max1(N))
    return TMM_ERR_LD;
  if (sA < 0 || sB < 0 || sC < 0) return TMM_ERR_STRIDE;
  if (M == 0 || N == 0 || batch == 0) {
    *quick = true;
    return TMM_OK;
  }
  if (batch > 1 && sC < (M - 1) * ldc + N) return TMM_ERR_STRIDE;
  if (C == nullptr) return TMM_ERR_NULL;
  if (K > 0 && (A == nullptr || B == nullptr)) return TMM_ERR_NULL;
  const int e = elem_bytes(ab);
  if (!aligned(C, elem_bytes(c)) || (bias && !aligned(bias, 4))) return TMM_ERR_ALIGN;
  if (K > 0 && (!aligned(A, e) || !aligned(B, e))) return TMM_ERR_ALIGN;
  // The grid has one workgroup per 128x128 tile or larger per problem.
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (tiles > (int64_t)0x7fffffff / batch) return TMM_ERR_DIM;
  // Kernels address A and B of one problem with 32-bit byte offsets.
  if (K > 0 && (((ex.trans_a ? (K - 1) * lda + M : (M - 1) * lda + K) * e) >= ((int64_t)1 << 32) ||
                ((trans_b ? (N - 1) * ldb + K : (K - 1) * ldb + N) * e) >= ((int64_t)1 << 32)))
    return TMM_ERR_DIM;
  return TMM_OK;
}

int cu_count() { return tmm::device_cu_count(); }

// Kernel-choice override for measurements and kernel-by-kernel tests, one
// setting for the whole library: TMM_OVERRIDE in the environment, parsed
// once at the first call, or tmm_set_override() at run time (include/tmm.h
// lists the keys).  Held as one packed word, so a call reads it with one
// atomic load and a setter never leaves a half-written value.
//   bits 0-7   tile choice + 1 (0: none): a tmm::Tile, or kOvGeneric,
//              kOvShortK, kOvGemvMulti
//   bits 8-15  skinny tile rows, 16-23 skinny tile columns (0: automatic)
//   bits 24-31 GEMV rows per wave, 32-39 GEMV waves per workgroup (0: automatic)
constexpr int kOvGeneric = 16, kOvShortK = 17, kOvGemvMulti = 18;
constexpr uint64_t kOvSet = 1ull << 63;

std::atomic<uint64_t> g_override{0};
std::once_flag g_override_env;

bool parse_override(const char *spec, uint64_t *out) {
  uint64_t v = kOvSet;
  if (!spec) {
    *out = v;
    return true;
  }
  char buf[256];
  if (strlen(spec) >= sizeof buf) return false;
  strcpy(buf, spec);
  char *save = nullptr;
  for (char *tok = strtok_r(buf, "; ", &save); tok; tok = strtok_r(nullptr, "; ", &save)) {
    char *eq = strchr(tok, '=');
    if (!eq) return false;
    *eq = 0;
    const char *key = tok, *val = eq + 1;
    if (!strcmp(key, "tile")) {
      static const struct { const char *name; int code; } names[] = {
          {"256x256", tmm::kTile256x256}, {"256x128", tmm::kTile256x128},
          {"128x128", tmm::kTile128x128}, {"256x256w4", tmm::kTile256x256w4},
          {"256x256s2", tmm::kTile256x256s2}, {"256x256r", tmm::kTile256x256r},
          {"256x256q", tmm::kTile256x256q}, {"256x128q", tmm::kTile256x128q},
          {"128x128q", tmm::kTile128x128q},
          {"skinny", tmm::kTileSkinny}, {"generic", kOvGeneric}, {"shortk", kOvShortK},
          {"gemvm", kOvGemvMulti}};
      int code = -1;
      for (const auto &n : names)
        if (!strcmp(val, n.name)) code = n.code;
      if (code < 0) return false;
      v = (v & ~0xffull) | (uint64_t)(code + 1);
    } else if (!strcmp(key, "skinny")) {
      int m = 0, n = 0;
      if (sscanf(val, "%dx%d", &m, &n) != 2 || (m != 16 && m != 32 && m != 64) ||
          (n != 16 && n != 32 && n != 64))
        return false;
      v = (v & ~(0xffffull << 8)) | ((uint64_t)m << 8) | ((uint64_t)n << 16);
    } else if (!strcmp(key, "gemv")) {
      int r = 0, w = 0;
      if (sscanf(val, "%dx%d", &r, &w) != 2 || (r != 1 && r != 2 && r != 4) ||
          (w != 4 && w != 8 && w != 16))
        return false;
      v = (v & ~(0xffffull << 24)) | ((uint64_t)r << 24) | ((uint64_t)w << 32);
    } else if (!strcmp(key, "conv")) {
      uint64_t c = 0;
      if (!strcmp(val, "quad")) c = 1;
      else if (!strcmp(val, "direct")) c = 2;
      else return false;
      v = (v & ~(3ull << 40)) | (c << 40);
    } else if (!strcmp(key, "ring")) {
      uint64_t c = 0;
      if (!strcmp(val, "4")) c = 1;
      else if (!strcmp(val, "8")) c = 2;
      else return false;
      v = (v & ~(3ull << 42)) | (c << 42);
    } else {
      return false;
    }
  }
  *out = v;
  return true;
}

uint64_t override_word() {
  std::call_once(g_override_env, [] {
    uint64_t v = kOvSet;
    if (!parse_override(getenv("TMM_OVERRIDE"), &v)) v = kOvSet;  // a bad value pins nothing
    uint64_t expect = 0;
    g_override.compare_exchange_strong(expect, v);
  });
  return g_override.load(std::memory_order_acquire);
}

int override_tile_code() { return (int)(override_word() & 0xff) - 1; }

// A pinned tmm::Tile shape, or -1.
int forced_tile() {
  const int c = override_tile_code();
  return c >= 0 && c < kOvGeneric ? c : -1;
}
bool forced_generic() { return override_tile_code() == kOvGeneric; }
bool forced_short_k() { return override_tile_code() == kOvShortK; }
bool forced_gemv_multi() { return override_tile_code() == kOvGemvMulti; }

// Largest M for which the several-row GEMV is chosen automatically: W 4096 x
// 4096 fp16 + bias, graph-timed, against the skinny MFMA kernel: M = 2
// 7.87 vs 8.81 us, M = 4 9.07 vs 9.17, M = 6 10.32 vs 9.44, M = 8 11.60 vs
// 9.99 (its dot instructions and LDS reads of X grow with M and run after
// the weight stream).  It takes up to 8 rows when forced.
constexpr int64_t kGemvMultiMaxM = 4;

// Largest M for which the skinny-M kernel is chosen automatically.
constexpr int64_t kSkinnyMaxM = 256;

// Skinny tile (bm, bn in 16 / 32 / 64): the least operand traffic into the
// CUs -- every tile reads its bm rows of A and its bn rows of B over all of
// K, i.e. K (M ceil(N/bn) + N ceil(M/bm)) elements -- among the shapes that
// give every CU a tile (the most tiles if none does).
void pick_skinny(int64_t M, int64_t N, int64_t batch, int *bm, int *bn) {
  // the override's "skinny=<bm>x<bn>" pins the tile
  const uint64_t ov = override_word();
  if ((ov >> 8) & 0xff) {
    *bm = (int)((ov >> 8) & 0xff);
    *bn = (int)((ov >> 16) & 0xff);
    return;
  }
  const int64_t cus = cu_count();
  double best = 1e300;
  int64_t best_tiles = -1;
  bool best_full = false;
  for (int m : {16, 32, 64}) {
    for (int n : {16, 32, 64}) {
      const int64_t tm = (M + m - 1) / m, tn = (N + n - 1) / n;
      const int64_t tiles = tm * tn * batch;
      const double traffic = (double)M * tn + (double)N * tm;
      const bool full = tiles >= cus;
      const bool better = full ? (!best_full || traffic < best)
                               : (!best_full && (tiles > best_tiles ||
                                                 (tiles == best_tiles && traffic < best)));
      if (better) {
        best = traffic;
        best_tiles = tiles;
        best_full = full;
        *bm = m;
        *bn = n;
      }
    }
  }
}

// Tile shape with the least estimated time: rounds of `cus` concurrent
// tiles times the work of one tile divided by the shape's relative MFMA
// efficiency (bigger tiles reuse each loaded byte more).
tmm::Tile pick_tile(int64_t M, int64_t N, int64_t batch, int ab) {
  const int f = forced_tile();
  if (f >= 0 && f != tmm::kTileSkinny) return (tmm::Tile)f;
  if (ab == TMM_F32) return tmm::kTile128x128;
  const int cus = cu_count();
  // One 128-column panel (N <= 128) with a long K, e.g. attention's P . V:
  // the product streams A from HBM and every tile shape reads the same
  // bytes.  For 16-bit inputs the four-wave kernel on 256x128 tiles streams
  // fastest (batch 128, 2048 x 128 x 2048 fp16, one box: 222 us against 235
  // on its 128x128 tiles, 243 on the two-stage 128x128 and 260 on the
  // two-stage 256x128; a six-stage ring on 256x128 gained nothing); the
  // others keep the two-stage 128x128 tiles, two workgroups per CU.
  if (N <= 128 && ab != TMM_F8E4M3 && ((M + 127) / 128) * batch >= 2 * (int64_t)cus)
    return (ab == TMM_BF16 || ab == TMM_F16) ? tmm::kTile256x128q : tmm::kTile128x128;
  const double eff[tmm::kNumAutoTiles] = {1.0, 0.85, 0.65};
  tmm::Tile best = tmm::kTile128x128;
  double best_cost = 1e300;
  for (int t = 0; t < tmm::kNumAutoTiles; ++t) {
    const int bm = tmm::tile_bm((tmm::Tile)t), bn = tmm::tile_bn((tmm::Tile)t);
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * batch;
    const int64_t rounds = (tiles + cus - 1) / cus;
    const double cost = (double)rounds * bm * bn / eff[t];
    if (cost < best_cost) {
      best_cost = cost;
      best = (tmm::Tile)t;
    }
  }
  // 16-bit inputs take the narrower tiles on the four-wave kernel (where
  // it applies; launch_tile falls back otherwise): 2048^3 NN bf16 33.1 ->
  // 23.3 us on 128x128, 1024 x 4096 x 4096 NT 48.8 -> 41.5 us, and equal at
  // 8192 x 1024 x 4096 NT on 256x128 (68.4 us).
  if (ab == TMM_BF16 || ab == TMM_F16) {
    if (best == tmm::kTile128x128) return tmm::kTile128x128q;
    if (best == tmm::kTile256x128) return tmm::kTile256x128q;
  }
  return best;
}

// Transposed A: the 256x256 ring kernel or the 64x64 any-layout kernel,
// by the same rounds-times-tile-work estimate as pick_tile (the any-layout
// kernel measured at about an eighth of the ring kernel's rate).  A forced
// "generic" takes the latter, a forced 256x256 shape the former.
bool use_ring_ta(int64_t M, int64_t N, int64_t batch) {
  const int f = forced_tile();
  if (f == tmm::kTile256x256 || f == tmm::kTile256x256r) return true;
  if (forced_generic()) return false;
  const int cus = cu_count();
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256) * batch;
  const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64) * batch;
  const double ring = (double)((t256 + cus - 1) / cus) * 256.0 * 256.0;
  const double gen = (double)((t64 + cus - 1) / cus) * 64.0 * 64.0 * 8.0;
  return ring <= gen;
}

// The persistent short-K kernel (gemm_short_k.hip): C = A . B^T, 16-bit in
// and out of one type, K = 64 or 128, whole 256x256 tiles, no bias, plain
// form, aligned rows and C.  Chosen automatically with at least four tiles
// per CU (a write-bound product: batched 2048 x 2048 x 128 fp16, the
// attention scores, 272 us on the two-stage kernel); "shortk" forces it.
bool short_k_ok(int64_t M, int64_t N, int64_t K, int ab, int c, int trans_b, int64_t lda, int64_t ldb,
                const void *C, int64_t ldc, int64_t sC, int64_t batch, const float *bias, bool plain,
                bool vec) {
  const int f = forced_tile();
  if (f >= 0 && !forced_short_k()) return false;
  if (!vec || !trans_b || !plain || bias || c != ab || (ab != TMM_BF16 && ab != TMM_F16)) return false;
  if ((K != 64 && K != 128) || M % 256 != 0 || N % 256 != 0) return false;
  if (!aligned(C, 16) || (ldc * 2) % 16 != 0 || (batch > 1 && (sC * 2) % 16 != 0)) return false;
  // the kernel's load offsets within a tile's 256 rows are 32-bit
  if (lda >= ((int64_t)1 << 22) || ldb >= ((int64_t)1 << 22)) return false;
  if (forced_short_k()) return true;
  return (M / 256) * (N / 256) * batch >= 4 * (int64_t)cu_count();
}

hipError_t dispatch_gemm(int ab, int c, bool trans_b, tmm::Tile tile, bool vec,
                         const tmm::GemmParams &p, hipStream_t s) {
  switch (ab) {
    case TMM_F32: return tmm::launch_gemm_f32((Fmt)c, trans_b, tile, vec, p, s);
    case TMM_BF16: return tmm::launch_gemm_bf16((Fmt)c, trans_b, tile, vec, p, s);
    case TMM_F16: return tmm::launch_gemm_f16((Fmt)c, trans_b, tile, vec, p, s);
    default: return tmm::launch_gemm_f8((Fmt)c, trans_b, tile, vec, p, s);
  }
}

int run_gemm(int64_t M, int64_t N, int64_t K, int ab, int c, int trans_b, const void *A,
             int64_t lda, int64_t sA, const void *B, int64_t ldb, int64_t sB, void *C, int64_t ldc,
             int64_t sC, int64_t batch, const float *bias, float scale_a, float scale_b,
             hipStream_t stream, const Ex &ex = Ex()) {
  bool quick = false;
  const int rc = check_gemm(M, N, K, ab, c, trans_b, A, lda, sA, B, ldb, sB, C, ldc, sC, batch,
                            bias, scale_a, scale_b, ex, &quick);
  if (rc != TMM_OK || quick) return rc;

  tmm::GemmParams p;
  p.M = M; p.N = N; p.K = K;
  p.A = A; p.lda = lda; p.strideA = sA;
  p.B = B; p.ldb = ldb; p.strideB = sB;
  p.C = C; p.ldc = ldc; p.strideC = sC;
  p.bias = bias;
  p.scale = scale_a * scale_b;
  p.batch = batch;
  p.beta = ex.beta;
  p.act = ex.act;
  const bool plain = p.scale == 1.f && p.beta == 0.f && p.act == 0;

  hipError_t err;
  if (K == 0) {
    err = tmm::launch_fill((Fmt)c, p, stream);
  } else if (ex.trans_a) {
    const int e = elem_bytes(ab);
    const bool va = aligned(A, 16) && (lda * e) % 16 == 0 && (batch == 1 || (sA * e) % 16 == 0);
    const bool vb = aligned(B, 16) && (ldb * e) % 16 == 0 && (batch == 1 || (sB * e) % 16 == 0);
    // the ring kernel reads whole 16-byte chunks of A's (and an NN B's)
    // k-rows and takes whole 32-element K-steps
    const bool ring_ok = va && vb && (M * e) % 16 == 0 && (trans_b || (N * e) % 16 == 0) && K % 32 == 0;
    if (ring_ok && use_ring_ta(M, N, batch))
      err = tmm::launch_gemm_ring_ta((Fmt)ab, (Fmt)c, trans_b != 0, p, stream);
    else
      err = tmm::launch_gemm_generic((Fmt)ab, (Fmt)c, true, trans_b != 0, va, vb, p, stream);
  } else if (M == 1 && batch == 1 && trans_b && ab != TMM_F8E4M3 && plain &&
             forced_tile() != tmm::kTileSkinny) {
    // y = W . x with W = B (N x K): the memory-bound matrix-vector path.
    tmm::GemvParams g;
    g.N = N; g.K = K; g.W = B; g.ldw = ldb; g.x = A; g.y = C; g.bias = bias;
    const int e = elem_bytes(ab);
    const bool vec = aligned(B, 16) && aligned(A, 16) && (ldb * e) % 16 == 0 && (K * e) % 16 == 0;
    err = tmm::launch_gemv((Fmt)ab, (Fmt)c, vec, g, stream);
  } else {
    const int e = elem_bytes(ab);
    // 16-byte loads need every row of A and B to start on a 16-byte boundary
    // (and the batch strides to keep it so); NN also needs N*e to be a
    // multiple of 16 so a 16-byte chunk of a B row is wholly inside or
    // outside N.
    const bool vec = aligned(A, 16) && aligned(B, 16) && (lda * e) % 16 == 0 &&
                     (ldb * e) % 16 == 0 &&
                     (batch == 1 || ((sA * e) % 16 == 0 && (sB * e) % 16 == 0)) &&
                     (trans_b || (N * e) % 16 == 0);
    const int f = forced_tile();
    const bool skinny_ok = vec && trans_b && (ab == TMM_BF16 || ab == TMM_F16);
    const bool generic_forced = forced_generic();
    // 16-byte loads, to registers and direct to LDS, return exact data at
    // 2-byte-aligned addresses too (measured on gfx950), and the tiled
    // kernels load a 16-byte chunk whole only when all of it lies inside the
    // operand (K tails and the chunk an NN B row's end cuts through go by
    // words, see load_words.h).  So 16-bit and fp32 operands need no more
    // than their element alignment for the tiled kernels (rows of
    // 1000 x 3000 x 777 or 4097 x 511 x 1023 bf16).  An NN B whose rows end
    // inside a 16-byte chunk (N * e % 16 != 0) stays off the ring kernel,
    // whose direct loads move whole chunks up to the last k-row; the
    // four-wave kernel takes it in its K-tail form (launch_tile), which
    // loads the last 64 k-rows itself, and the two-stage kernel where that
    // form does not apply.
    const bool elem16 = ab == TMM_BF16 || ab == TMM_F16 || ab == TMM_F32;
    const bool loads16 = vec || elem16;
    const bool nn_cut = !trans_b && (N * e) % 16 != 0;
    const bool ragged_nn = !loads16 && !trans_b && f < 0 && (ab == TMM_BF16 || ab == TMM_F16);
    if ((generic_forced || ragged_nn) && (ab == TMM_BF16 || ab == TMM_F16)) {
      const int e = elem_bytes(ab);
      const bool va = aligned(A, 16) && (lda * e) % 16 == 0 && (batch == 1 || (sA * e) % 16 == 0);
      const bool vb = aligned(B, 16) && (ldb * e) % 16 == 0 && (batch == 1 || (sB * e) % 16 == 0);
      err = tmm::launch_gemm_generic((Fmt)ab, (Fmt)c, false, trans_b != 0, va, vb, p, stream);
    } else if (vec && trans_b && plain && batch == 1 && (ab == TMM_BF16 || ab == TMM_F16) &&
               M >= 2 && M <= 8 && (K * e) % 16 == 0 &&
               (forced_gemv_multi() || (f < 0 && M <= kGemvMultiMaxM))) {
      // Y = X . W^T for a few rows X: the weight stream of the GEMV with M
      // dot products per weight chunk.
      tmm::GemvMParams g;
      g.N = N; g.K = K; g.W = B; g.ldw = ldb; g.x = A; g.ldx = lda; g.M = M;
      g.y = C; g.ldy = ldc; g.bias = bias;
      err = tmm::launch_gemv_multi((Fmt)ab, (Fmt)c, g, stream);
    } else if (short_k_ok(M, N, K, ab, c, trans_b, lda, ldb, C, ldc, sC, batch, bias, plain, vec)) {
      const int64_t total = (M / 256) * (N / 256) * batch;
      const int64_t cus = cu_count();
      const unsigned grid = (unsigned)std::max<int64_t>(8, std::min<int64_t>(total, cus) / 8 * 8);
      err = tmm::launch_gemm_short_k((Fmt)ab, p, grid, stream);
    } else if (skinny_ok && !ex.no_skinny && (f == tmm::kTileSkinny || (f < 0 && M <= kSkinnyMaxM))) {
      int bm, bn;
      pick_skinny(M, N, batch, &bm, &bn);
      const int ce = elem_bytes(c);
      const bool vec_c = aligned(C, 4 * ce) && ldc % 4 == 0 && (batch == 1 || sC % 4 == 0);
      err = tmm::launch_gemm_skinny((Fmt)ab, (Fmt)c, bm, bn, vec_c, p, stream);
    } else if (ab == TMM_F32 && f < 0 && !generic_forced &&
               ((M + 127) / 128) * ((N + 127) / 128) * batch * 2 <= cu_count()) {
      // fp32 with at most one 128x128 tile per two CUs: 32x32 tiles with K
      // split over a workgroup's waves (fp32 256^3: 21.2 us on four 128x128
      // tiles)
      err = tmm::launch_gemm_f32_small(trans_b != 0, p, stream);
    } else {
      tmm::Tile tile = loads16 ? pick_tile(M, N, batch, ab) : tmm::kTile128x128;
      if (nn_cut && tile == tmm::kTile256x256r) tile = tmm::kTile256x256s2;  // the ring needs whole NN B chunks
      err = dispatch_gemm(ab, c, trans_b != 0, tile, loads16, p, stream);
    }
  }
  return err == hipSuccess ? TMM_OK : TMM_ERR_LAUNCH;
}

// Checks shared by the two split-K entry points; *done when the call is
// complete without the split (a quick return, or splits == 1 / K == 0: the
// one-pass product, enqueued here).
int check_splitk(int64_t M, int64_t N, int64_t K, int ab, int c, int trans_b, const void *A,
                 int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc, const float *bias,
                 float scale_a, float scale_b, int splits, hipStream_t stream, bool *done) {
  *done = false;
  if (splits < 1 || splits > 64) return TMM_ERR_ARG;
  bool quick = false;
  const int rc = check_gemm(M, N, K, ab, c, trans_b, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, bias,
                            scale_a, scale_b, Ex(), &quick);
  if (rc != TMM_OK) return rc;
  if (K % splits != 0) return TMM_ERR_ARG;
  if (quick) {
    *done = true;
    return TMM_OK;
  }
  if (splits == 1 || K == 0) {
    *done = true;
    return run_gemm(M, N, K, ab, c, trans_b, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, bias, scale_a,
                    scale_b, stream);
  }
  return TMM_OK;
}

// Split-K product (arguments checked by the caller): the K slices as one
// batched fp32 product into W (slice s = batch entry s: A and B advanced by
// K/S along K, W[s] dense M x N), kept off the skinny kernel so that the
// tile choice sees S x the tiles, then the fixed-order sum with scale, bias
// and one rounding (splitk.hip).
int run_splitk(int64_t M, int64_t N, int64_t K, int ab, int c, int trans_b, const void *A,
               int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc, const float *bias,
               float scale_a, float scale_b, int splits, float *W, hipStream_t stream) {
  Ex ex;
  ex.no_skinny = true;
  const int64_t ks = K / splits;
  const int rc = run_gemm(M, N, ks, ab, TMM_F32, trans_b, A, lda, ks, B, ldb, trans_b ? ks : ks * ldb,
                          W, N, M * N, splits, nullptr, 1.0f, 1.0f, stream, ex);
  if (rc != TMM_OK) return rc;
  const hipError_t err = tmm::launch_splitk_reduce((Fmt)c, M, N, splits, W, C, ldc, bias,
                                                   scale_a * scale_b, stream);
  return err == hipSuccess ? TMM_OK : TMM_ERR_LAUNCH;
}

}  // namespace

// Scratch of tmm_gemm_splitk_noalloc: the split-K partial products of calls
// that bring no workspace.  One copy per GPU (device memory of the code
// object, zero-initialised at load, held until the process ends); nothing
// in it needs to start at zero, as every call overwrites the partials it
// reads.  Host code never uses this name as an address: scratch_address()
// gives the current device's copy.
constexpr int64_t kScratchBytes = TMM_SPLITK_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// Device address of this device's `scratch`, looked up with that device
// current (hipGetSymbolAddress) at the first call on it and kept;
// TMM_ERR_LAUNCH when the device or the lookup fails (tried again next call).
int scratch_address(void **out) {
  static std::mutex mu;
  static void *addr[64] = {nullptr};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return TMM_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TMM_ERR_LAUNCH;
    addr[dev] = p;
  }
  *out = addr[dev];
  return TMM_OK;
}

}  // namespace

extern "C" {

int tmm_gemm(int64_t M, int64_t N, int64_t K, tmm_dtype ab_type, tmm_dtype c_type, int trans_b,
             const void *A, int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
             const float *bias, float scale_a, float scale_b, hipStream_t stream) {
  return run_gemm(M, N, K, ab_type, c_type, trans_b, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, bias,
                  scale_a, scale_b, stream);
}

int tmm_gemm_ex(int64_t M, int64_t N, int64_t K, tmm_dtype ab_type, tmm_dtype c_type,
                int trans_a, int trans_b, const void *A, int64_t lda, int64_t strideA,
                const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc,
                int64_t strideC, int64_t batch, const float *bias, float alpha, float beta,
                int activation, hipStream_t stream) {
  Ex ex;
  ex.full = true;
  ex.trans_a = trans_a != 0;
  ex.beta = beta;
  ex.act = activation;
  return run_gemm(M, N, K, ab_type, c_type, trans_b, A, lda, strideA, B, ldb, strideB, C, ldc,
                  strideC, batch, bias, alpha, 1.0f, stream, ex);
}

int tmm_gemm_strided_batched(int64_t M, int64_t N, int64_t K, tmm_dtype ab_type,
                             tmm_dtype c_type, int trans_b, const void *A, int64_t lda,
                             int64_t strideA, const void *B, int64_t ldb, int64_t strideB, void *C,
                             int64_t ldc, int64_t strideC, int64_t batch, const float *bias,
                             float scale_a, float scale_b, hipStream_t stream) {
  return run_gemm(M, N, K, ab_type, c_type, trans_b, A, lda, strideA, B, ldb, strideB, C, ldc,
                  strideC, batch, bias, scale_a, scale_b, stream);
}

int tmm_gemm_splitk(int64_t M, int64_t N, int64_t K, tmm_dtype ab_type, tmm_dtype c_type,
                    int trans_b, const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                    int64_t ldc, const float *bias, float scale_a, float scale_b, int splits,
                    void *workspace, int64_t workspace_bytes, hipStream_t stream) {
  bool done = false;
  const int rc = check_splitk(M, N, K, ab_type, c_type, trans_b, A, lda, B, ldb, C, ldc, bias,
                              scale_a, scale_b, splits, stream, &done);
  if (rc != TMM_OK || done) return rc;
  // M * N < 2^62 / 256 here (check_gemm bounds the tiles), so no overflow
  const int64_t need = (int64_t)splits * M * N * 4;
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return TMM_ERR_WORKSPACE;
  return run_splitk(M, N, K, ab_type, c_type, trans_b, A, lda, B, ldb, C, ldc, bias, scale_a,
                    scale_b, splits, (float *)workspace, stream);
}

int tmm_gemm_splitk_noalloc(int64_t M, int64_t N, int64_t K, tmm_dtype ab_type, tmm_dtype c_type,
                            int trans_b, const void *A, int64_t lda, const void *B, int64_t ldb,
                            void *C, int64_t ldc, const float *bias, float scale_a, float scale_b,
                            int splits, hipStream_t stream) {
  bool done = false;
  const int rc = check_splitk(M, N, K, ab_type, c_type, trans_b, A, lda, B, ldb, C, ldc, bias,
                              scale_a, scale_b, splits, stream, &done);
  if (rc != TMM_OK || done) return rc;
  const int64_t need = (int64_t)splits * M * N * 4;
  if (need > kScratchBytes) return TMM_ERR_WORKSPACE;
  void *ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != TMM_OK) return st;
  return run_splitk(M, N, K, ab_type, c_type, trans_b, A, lda, B, ldb, C, ldc, bias, scale_a,
                    scale_b, splits, (float *)ws, stream);
}

int tmm_gemv(int64_t N, int64_t K, tmm_dtype w_type, tmm_dtype y_type, const void *W,
             int64_t ldw, const void *x, void *y, const float *bias, hipStream_t stream) {
  if (N < 0 || K < 0) return TMM_ERR_DIM;
  if (!known_type(w_type) || !known_type(y_type) || w_type == TMM_F8E4M3 ||
      !pair_ok(w_type, y_type))
    return TMM_ERR_DTYPE;
  if (ldw < max1(K)) return TMM_ERR_LD;
  if (N == 0) return TMM_OK;
  if (y == nullptr) return TMM_ERR_NULL;
  if (K > 0 && (W == nullptr || x == nullptr)) return TMM_ERR_NULL;
  const int e = elem_bytes(w_type);
  if (!aligned(y, elem_bytes(y_type)) || (bias && !aligned(bias, 4))) return TMM_ERR_ALIGN;
  if (K > 0 && (!aligned(W, e) || !aligned(x, e))) return TMM_ERR_ALIGN;
  if (N > (int64_t)0x7fffffff) return TMM_ERR_DIM;

  hipError_t err;
  if (K == 0) {
    tmm::GemmParams p;
    memset(&p, 0, sizeof p);
    p.M = 1; p.N = N; p.K = 0; p.C = y; p.ldc = N; p.bias = bias; p.batch = 1; p.scale = 1.f;
    err = tmm::launch_fill((Fmt)y_type, p, stream);
  } else {
    tmm::GemvParams g;
    g.N = N; g.K = K; g.W = W; g.ldw = ldw; g.x = x; g.y = y; g.bias = bias;
    const bool vec = aligned(W, 16) && aligned(x, 16) && (ldw * e) % 16 == 0 && (K * e) % 16 == 0;
    err = tmm::launch_gemv((Fmt)w_type, (Fmt)y_type, vec, g, stream);
  }
  return err == hipSuccess ? TMM_OK : TMM_ERR_LAUNCH;
}

// Largest K / V leading dimension of the attention kernel (elements).
constexpr int64_t kMaxAttnLd = (int64_t)1 << 24;

int tmm_attention_fwd(int64_t batch, int64_t Nq, int64_t Nk, int64_t D, tmm_dtype in_type,
                      tmm_dtype out_type, const void *Q, int64_t ldq, int64_t strideQ,
                      const void *K, int64_t ldk, int64_t strideK, const void *V, int64_t ldv,
                      int64_t strideV, void *O, int64_t ldo, int64_t strideO, float scale,
                      hipStream_t stream) {
  if (batch < 0 || Nq < 0 || Nk < 0 || (D != 64 && D != 128)) return TMM_ERR_DIM;
  if ((in_type != TMM_F16 && in_type != TMM_BF16) ||
      (out_type != in_type && out_type != TMM_F32))
    return TMM_ERR_DTYPE;
  if (ldq < D || ldk < D || ldv < D || ldo < D) return TMM_ERR_LD;
  if (ldk > kMaxAttnLd || ldv > kMaxAttnLd) return TMM_ERR_LD;  // 32-bit offsets within a key block
  if (strideQ < 0 || strideK < 0 || strideV < 0 || strideO < 0) return TMM_ERR_STRIDE;
  if (batch > 1 && Nq > 0 && strideO < (Nq - 1) * ldo + D) return TMM_ERR_STRIDE;
  const float scale_log2 = scale * 1.4426950408889634f;   // exponentials are base 2
  if (!isfinite(scale) || !isfinite(scale_log2)) return TMM_ERR_SCALE;
  if (batch == 0 || Nq == 0) return TMM_OK;
  if (Nk == 0) return TMM_ERR_DIM;  // softmax over no keys
  if (!Q || !K || !V || !O) return TMM_ERR_NULL;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || ldq % 8 ||
      ldk % 8 || ldv % 8 || ldo % 8 || strideQ % 8 || strideK % 8 || strideV % 8 || strideO % 8)
    return TMM_ERR_ALIGN;
  if (batch * ((Nq + 127) / 128) >= ((int64_t)1 << 31)) return TMM_ERR_DIM;

  tmm::AttnParams p;
  p.Z = batch; p.Nq = Nq; p.Nk = Nk;
  p.Q = Q; p.ldq = ldq; p.strideQ = strideQ;
  p.K = K; p.ldk = ldk; p.strideK = strideK;
  p.V = V; p.ldv = ldv; p.strideV = strideV;
  p.O = O; p.ldo = ldo; p.strideO = strideO;
  p.scale_log2 = scale_log2;
  const hipError_t err = tmm::launch_attention((Fmt)in_type, (Fmt)out_type, (int)D, p, stream);
  return err == hipSuccess ? TMM_OK : TMM_ERR_LAUNCH;
}

int tmm_conv2d_fused(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                     int64_t pad, tmm_dtype in_type, tmm_dtype out_type, const void *in,
                     const void *w, const float *scale, const float *bias, int activation,
                     int pool, void *out, hipStream_t stream) {
  const int64_t big = (int64_t)1 << 31;
  if (N < 0 || H < 1 || W < 1 || C < 1 || K < 1 || R < 1 || S < 1 || pad < 0) return TMM_ERR_DIM;
  if (H >= big || W >= big || C >= big || K >= big || R >= big || S >= big || pad >= big ||
      R * S * C >= big)
    return TMM_ERR_DIM;
  if ((in_type != TMM_BF16 && in_type != TMM_F16) || (out_type != in_type && out_type != TMM_F32))
    return TMM_ERR_DTYPE;
  if (activation != TMM_ACT_NONE && activation != TMM_ACT_RELU) return TMM_ERR_ARG;
  if (pool != 1 && pool != 2) return TMM_ERR_ARG;
  const int64_t P = H + 2 * pad - R + 1, Q = W + 2 * pad - S + 1;
  if (P < 1 || Q < 1 || (pool == 2 && (P % 2 || Q % 2))) return TMM_ERR_DIM;
  if (N == 0) return TMM_OK;
  if (!in || !w || !out) return TMM_ERR_NULL;
  if (C % 8 || !aligned(in, 16) || !aligned(w, 16) || !aligned(out, elem_bytes(out_type)) ||
      (scale && !aligned(scale, 4)) || (bias && !aligned(bias, 4)))
    return TMM_ERR_ALIGN;
  const int64_t tiles = ((N * P * Q + 127) / 128) * ((K + 63) / 64);
  if (N * P * Q >= ((int64_t)1 << 40) || tiles >= big) return TMM_ERR_DIM;

  tmm::ConvParams p;
  p.N = N; p.H = (int)H; p.W = (int)W; p.C = (int)C; p.K = (int)K; p.R = (int)R; p.S = (int)S;
  p.pad = (int)pad; p.pool = pool; p.relu = activation == TMM_ACT_RELU ? 1 : 0;
  p.in = in; p.w = w; p.scale = scale; p.bias = bias; p.out = out;
  const hipError_t err = tmm::launch_conv((Fmt)in_type, (Fmt)out_type, p, stream);
  return err == hipSuccess ? TMM_OK : TMM_ERR_LAUNCH;
}

const char *tmm_status_string(int status) {
  switch (status) {
    case TMM_OK: return "success";
    case TMM_ERR_DIM: return "negative or too large dimension or batch";
    case TMM_ERR_LD: return "leading dimension smaller than the row length";
    case TMM_ERR_NULL: return "null pointer for an operand with non-zero extent";
    case TMM_ERR_DTYPE: return "unsupported element type or type combination";
    case TMM_ERR_SCALE: return "scale, alpha or beta not finite, or a scale != 1 for non-fp8 inputs";
    case TMM_ERR_STRIDE: return "negative batch stride or overlapping output matrices";
    case TMM_ERR_ALIGN: return "pointer not aligned to its element size";
    case TMM_ERR_LAUNCH: return "HIP reported an error at kernel launch";
    case TMM_ERR_ARG: return "unknown activation code or pooling factor, or a split count outside 1..64 or not dividing K";
    case TMM_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    default: return "unknown status code";
  }
}

int tmm_version(void) { return kVersion; }

int tmm_set_override(const char *spec) {
  uint64_t v = 0;
  if (!parse_override(spec, &v)) return TMM_ERR_ARG;
  override_word();  // the environment's value is read first, then replaced
  g_override.store(v, std::memory_order_release);
  return TMM_OK;
}

}  // extern "C"
