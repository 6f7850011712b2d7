/* Test-only build aid for the CPU oracle (tests/test_oracle_uninit.py): every
 * block from malloc starts as 0xFF bytes, which read as NaN for floats and
 * doubles and as 0xFFFFFFFF for indices.  An oracle result that depends on
 * memory read before it is written then shows (non-finite values, different
 * bits, or an out-of-range index). */
#ifndef LAPLEX_ORACLE_POISON_H
#define LAPLEX_ORACLE_POISON_H
#include <stdlib.h>
#include <string.h>
static inline void* lo_poisoned_malloc(size_t n) {
  void* p = malloc(n);
  if (p) memset(p, 0xFF, n);
  return p;
}
#define malloc(n) lo_poisoned_malloc(n)
#endif
