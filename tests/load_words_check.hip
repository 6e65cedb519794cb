// CPU check of load8_u16_words and load8_u16_tail (tiled_matrix_multiplication_amd/csrc/load_words.h),
// built for the host only and run by tests/test_load_words.py.
//
// For both alignments h (p on a 4-byte boundary, or 2 bytes past one) and
// every count nv = 0 .. 8 of valid elements, the 8-element window is placed
// so that the 4-byte word holding element nv - 1 ends exactly where a
// PROT_NONE guard page begins (for nv = 0: p itself sits at the guard page).
// A read of any later word faults, so a clean exit shows the helper touches
// nothing past the last valid element's word.  The values are checked too:
// elements 0 .. nv-1 as stored, zero after.
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <sys/mman.h>
#include <unistd.h>

#include "load_words.h"

int main() {
  const long page = sysconf(_SC_PAGESIZE);
  char *base = (char *)mmap(nullptr, 2 * page, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
  if (base == MAP_FAILED) return 2;
  char *guard = base + page;
  // element values: 0x1000 + byte offset / 2, so every position is distinct
  for (long i = 0; i < page / 2; ++i) ((uint16_t *)base)[i] = (uint16_t)(0x1000 + i);
  if (mprotect(guard, page, PROT_NONE) != 0) return 3;
  int checked = 0;
  for (int h = 0; h <= 1; ++h) {
    for (int nv = 0; nv <= 8; ++nv) {
      // byte offset (from the word boundary q) of the end of the word holding element nv - 1
      const long end = nv == 0 ? 2 * h : ((2 * h + 2 * (nv - 1)) / 4 + 1) * 4;
      const char *q = guard - end;
      const char *p = q + 2 * h;
      const tmm::lw_i32x4 v = tmm::load8_u16_words(p, nv);
      uint16_t got[8];
      for (int w = 0; w < 4; ++w) {
        got[2 * w] = (uint16_t)((uint32_t)v[w] & 0xffffu);
        got[2 * w + 1] = (uint16_t)((uint32_t)v[w] >> 16);
      }
      for (int e = 0; e < 8; ++e) {
        const uint16_t want = e < nv ? ((const uint16_t *)p)[e] : 0;
        if (got[e] != want) {
          printf("FAIL h=%d nv=%d element %d: got 0x%04x want 0x%04x\n", h, nv, e, got[e], want);
          return 1;
        }
      }
      ++checked;
    }
  }
  // whole, interior windows at both alignments: every element as stored
  for (int h = 0; h <= 1; ++h) {
    const char *p = base + 64 + 2 * h;
    const tmm::lw_i32x4 v = tmm::load8_u16_words(p, 8);
    for (int e = 0; e < 8; ++e) {
      const uint16_t g = (uint16_t)((uint32_t)v[e / 2] >> (16 * (e & 1)));
      if (g != ((const uint16_t *)p)[e]) {
        printf("FAIL interior h=%d element %d\n", h, e);
        return 1;
      }
    }
    ++checked;
  }
  // load8_u16_tail: one 16-byte read ending at the last valid element, or,
  // for nv == 0, the valid chunk at p; the read ends exactly at the guard
  // page, so reading one byte more faults.  p = guard - 2 nv takes every
  // 2-byte alignment modulo 16 as nv runs over 1 .. 8.
  for (int nv = 0; nv <= 8; ++nv) {
    const char *p = nv == 0 ? guard - 16 : guard - 2 * nv;
    const tmm::lw_i32x4 v = tmm::load8_u16_tail(p, nv);
    for (int e = 0; e < 8; ++e) {
      const uint16_t g = (uint16_t)((uint32_t)v[e / 2] >> (16 * (e & 1)));
      const uint16_t want = e < nv ? ((const uint16_t *)p)[e] : 0;
      if (g != want) {
        printf("FAIL tail nv=%d element %d: got 0x%04x want 0x%04x\n", nv, e, g, want);
        return 1;
      }
    }
    ++checked;
  }
  printf("OK %d windows\n", checked);
  munmap(base, 2 * page);
  return 0;
}
