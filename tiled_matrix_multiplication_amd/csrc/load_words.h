// Misaligned 16-bit row pieces read as 4-byte words, shared by the kernels
// that accept rows which are not 16-byte aligned (the edge-tile and
// alignment handling of the "GEMM to FlashAttention" page's tiled_matmul
// min() bounds and the devpress notes' section 3.6 on aligned accesses).
// Host-callable as well, so the exact set of words it touches is checked on
// the CPU against a guard page.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tmm {

typedef int lw_i32x4 __attribute__((ext_vector_type(4)));

// Elements [0, nv) of the 8 consecutive 16-bit elements at p (2-byte
// aligned), zero past them (0 <= nv <= 8), read as 4-byte words from the
// word boundary at or below p: word j holds elements 2j - h and 2j - h + 1
// (h = 1 when p is two bytes past a boundary); it is read only when one of
// them is valid, so no word past the one holding element nv - 1 is touched
// (and none when nv == 0).  Each output word is the 16-bit funnel shift of
// two neighbours: 5 word loads instead of 8 two-byte loads, the same
// instructions for every alignment.
__host__ __device__ __forceinline__ lw_i32x4 load8_u16_words(const char *p, int nv) {
  const int h = (int)(((uintptr_t)p >> 1) & 1);
  const uint32_t *q = (const uint32_t *)(p - 2 * h);
  uint32_t d[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int lo = 2 * j - h > 0 ? 2 * j - h : 0;
    const bool ok = lo < nv && lo <= 2 * j - h + 1 && lo <= 7;
    d[j] = ok ? q[j] : 0u;
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = (uint32_t)((((uint64_t)d[i + 1] << 32) | d[i]) >> (16 * h));
    o[i] = 2 * i >= nv ? 0u : (2 * i + 1 < nv ? w : (w & 0xffffu));
  }
  return lw_i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

}  // namespace tmm
