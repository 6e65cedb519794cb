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

// Elements [0, nv) of the 8 consecutive 16-bit elements at p, zero past them
// (0 <= nv <= 8), with one 16-byte load and no branch: for 0 < nv < 8 it
// loads the 8 elements that end at element nv - 1 (from p - 2 (8 - nv)) and
// shifts them down by 8 - nv elements; for nv == 0 it loads at p and keeps
// nothing.  The caller guarantees that those 16 bytes lie inside the operand
// (for the chunk a row's end cuts through: the row holds at least 8
// elements; for nv == 0: p is a valid chunk).  16-byte loads at 2-byte
// alignment return exact data on gfx950 (measured), so the kernels use one
// plain load where load8_u16_words would use five and a branch per lane.
// Split in two so a kernel can issue the load early and shift when it uses
// the data: tail_load_addr gives the address, tail_shift the result.
__host__ __device__ __forceinline__ const char *tail_load_addr(const char *p, int nv) {
  return p - 2 * (nv > 0 ? 8 - nv : 0);
}

__host__ __device__ __forceinline__ lw_i32x4 tail_shift(const lw_i32x4 &v, int nv) {
  const int s = nv > 0 ? 8 - nv : 0;  // elements shifted out at the bottom
  const int w = s >> 1, h = s & 1;
  uint32_t e[5];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // dword i + w of v, or zero past the end (a select chain, no indexing)
    const int k = i + w;
    e[i] = k == 0 ? (uint32_t)v[0] : k == 1 ? (uint32_t)v[1] : k == 2 ? (uint32_t)v[2] : k == 3 ? (uint32_t)v[3] : 0u;
  }
  e[4] = 0u;
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = h ? ((e[i] >> 16) | (e[i + 1] << 16)) : e[i];
    // keep elements 2i, 2i + 1 only below nv
    o[i] = 2 * i >= nv ? 0u : (2 * i + 1 < nv ? x : (x & 0xffffu));
  }
  return lw_i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

__host__ __device__ __forceinline__ lw_i32x4 load8_u16_tail(const char *p, int nv) {
  lw_i32x4 v;
#if defined(__HIP_DEVICE_COMPILE__)
  v = *(const lw_i32x4 *)tail_load_addr(p, nv);
#else
  __builtin_memcpy(&v, tail_load_addr(p, nv), 16);  // host: no alignment assumed
#endif
  return tail_shift(v, nv);
}

}  // namespace tmm
