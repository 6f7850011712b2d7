/*
 * LAPLEX CPU oracle on all host cores -- TEST INFRASTRUCTURE ONLY.
 *
 * The symmetric operator y = K(a, a) x, K_ij = exp(-|a_i - a_j|), by the
 * scan algebra of "LAPLEX: The FFT of Learnable Laplace Kernels" (technical
 * summary, section 2.2 "Exact Scan Algebra": sort the anchors, then a prefix
 * scan L_i = x_i + exp(a_{i-1} - a_i) L_{i-1} and the mirrored suffix scan U,
 * and y = L + U - x in sorted order), in float64, spread over OpenMP threads:
 *
 *   sort:  each thread sorts a contiguous block of (anchor, index) pairs by a
 *          bottom-up merge sort, then the blocks are merged pairwise, each
 *          merge split among the threads along its merge path.  Pairs are
 *          ordered by anchor and then by index, so the order is the stable
 *          ascending argsort whatever the merge order (-0.0 equals +0.0).
 *   scan:  the sorted sequence is cut into one chunk per thread.  Pass 1
 *          folds each chunk with no carry in; the chunk carries are joined
 *          one after another (L at the end of chunk k is its fold plus
 *          exp(a_before - a_last) times the carry entering it); pass 2 runs
 *          both recurrences again from the carries and writes y.
 *
 * The one-core oracle (laplex_oracle.c) is the reference this file is
 * checked against; the two share no code.  Returns 0, -1 for a non-finite
 * anchor, -2 when out of memory.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  float v;
  uint32_t i;
} pair_t;

static inline int before(pair_t p, pair_t q) { return p.v < q.v || (p.v == q.v && p.i < q.i); }

static void merge_into(const pair_t* A, int64_t na, const pair_t* B, int64_t nb, pair_t* C) {
  int64_t p = 0, q = 0, o = 0;
  while (p < na && q < nb) C[o++] = before(B[q], A[p]) ? B[q++] : A[p++];
  while (p < na) C[o++] = A[p++];
  while (q < nb) C[o++] = B[q++];
}

/* number of A elements among the first d of the merge of A and B */
static int64_t merge_path(const pair_t* A, int64_t na, const pair_t* B, int64_t nb, int64_t d) {
  int64_t lo = d > nb ? d - nb : 0, hi = d < na ? d : na;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (before(A[mid], B[d - mid - 1]))
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

static void block_sort(pair_t* v, pair_t* tmp, int64_t n) {
  for (int64_t w = 1; w < n; w *= 2) {
    for (int64_t lo = 0; lo < n; lo += 2 * w) {
      const int64_t mid = lo + w < n ? lo + w : n, hi = lo + 2 * w < n ? lo + 2 * w : n;
      merge_into(v + lo, mid - lo, v + mid, hi - mid, tmp + lo);
    }
    memcpy(v, tmp, sizeof(pair_t) * (size_t)n);
  }
}

static int par_argsort(const float* a, int64_t n, pair_t* out, int T) {
  pair_t* buf = (pair_t*)malloc(sizeof(pair_t) * (size_t)n);
  pair_t* tmp = (pair_t*)malloc(sizeof(pair_t) * (size_t)n);
  if (!buf || !tmp) {
    free(buf);
    free(tmp);
    return -2;
  }
  int bad = 0;
#pragma omp parallel for num_threads(T) reduction(| : bad)
  for (int64_t i = 0; i < n; ++i) {
    bad |= !isfinite(a[i]);
    buf[i].v = a[i] == 0.0f ? 0.0f : a[i];
    buf[i].i = (uint32_t)i;
  }
  if (bad) {
    free(buf);
    free(tmp);
    return -1;
  }
  const int64_t blk = (n + T - 1) / T;
#pragma omp parallel for num_threads(T) schedule(static, 1)
  for (int t = 0; t < T; ++t) {
    const int64_t lo = (int64_t)t * blk, hi = lo + blk < n ? lo + blk : n;
    if (lo < hi) block_sort(buf + lo, tmp + lo, hi - lo);
  }
  /* pairwise merges of sorted runs of width w, each split along its merge path */
  pair_t *src = buf, *dst = tmp;
  for (int64_t w = blk; w < n; w *= 2) {
    for (int64_t lo = 0; lo < n; lo += 2 * w) {
      const int64_t mid = lo + w < n ? lo + w : n, hi = lo + 2 * w < n ? lo + 2 * w : n;
      const pair_t* A = src + lo;
      const pair_t* B = src + mid;
      const int64_t na = mid - lo, nb = hi - mid, tot = na + nb;
#pragma omp parallel for num_threads(T) schedule(static, 1)
      for (int t = 0; t < T; ++t) {
        const int64_t d0 = tot * t / T, d1 = tot * (t + 1) / T;
        const int64_t i0 = merge_path(A, na, B, nb, d0), i1 = merge_path(A, na, B, nb, d1);
        merge_into(A + i0, i1 - i0, B + (d0 - i0), (d1 - i1) - (d0 - i0), dst + lo + d0);
      }
    }
    pair_t* s = src;
    src = dst;
    dst = s;
  }
  memcpy(out, src, sizeof(pair_t) * (size_t)n);
  free(buf);
  free(tmp);
  return 0;
}

int lop_threads(void) { return omp_get_max_threads(); }

/* perm (n) receives the stable ascending argsort of a */
int lop_stable_argsort(const float* a, int64_t n, uint32_t* perm) {
  if (n <= 0) return 0;
  pair_t* s = (pair_t*)malloc(sizeof(pair_t) * (size_t)n);
  if (!s) return -2;
  const int rc = par_argsort(a, n, s, omp_get_max_threads());
  if (rc == 0) {
#pragma omp parallel for
    for (int64_t i = 0; i < n; ++i) perm[i] = s[i].i;
  }
  free(s);
  return rc;
}

/* y (n x m, float64, original order) = K(a, a) x, x row-major n x m */
int lop_sym_apply(const float* a, int64_t n, int64_t m, const float* x, double* y) {
  if (n <= 0 || m <= 0) return 0;
  const int T = omp_get_max_threads();
  pair_t* s = (pair_t*)malloc(sizeof(pair_t) * (size_t)n);
  double* L = (double*)malloc(sizeof(double) * (size_t)n * (size_t)m);
  double* agg = (double*)malloc(sizeof(double) * (size_t)(4 * T) * (size_t)m); /* fwd, bwd folds; fwd, bwd carries */
  if (!s || !L || !agg) {
    free(s);
    free(L);
    free(agg);
    return -2;
  }
  int rc = par_argsort(a, n, s, T);
  if (rc != 0) {
    free(s);
    free(L);
    free(agg);
    return rc;
  }
  const int64_t ch = (n + T - 1) / T;
  double* fold_f = agg;
  double* fold_b = agg + (size_t)T * m;
  double* carry_f = agg + (size_t)2 * T * m; /* L at the element before the chunk */
  double* carry_b = agg + (size_t)3 * T * m; /* U at the element after the chunk */
  /* pass 1: folds with no carry in */
#pragma omp parallel for num_threads(T) schedule(static, 1)
  for (int t = 0; t < T; ++t) {
    const int64_t lo = (int64_t)t * ch, hi = lo + ch < n ? lo + ch : n;
    for (int64_t c = 0; c < m; ++c) {
      double f = 0.0, b = 0.0;
      for (int64_t i = lo; i < hi; ++i)
        f = (double)x[(size_t)s[i].i * m + c] + (i > lo ? exp((double)s[i - 1].v - (double)s[i].v) : 0.0) * f;
      for (int64_t i = hi - 1; i >= lo; --i)
        b = (double)x[(size_t)s[i].i * m + c] + (i < hi - 1 ? exp((double)s[i].v - (double)s[i + 1].v) : 0.0) * b;
      fold_f[(size_t)t * m + c] = f;
      fold_b[(size_t)t * m + c] = b;
    }
  }
  /* carries, chunk by chunk */
  for (int64_t c = 0; c < m; ++c) {
    double cf = 0.0;
    for (int t = 0; t < T; ++t) {
      const int64_t lo = (int64_t)t * ch, hi = lo + ch < n ? lo + ch : n;
      carry_f[(size_t)t * m + c] = cf;
      if (lo < hi) cf = fold_f[(size_t)t * m + c] + (lo > 0 ? exp((double)s[lo - 1].v - (double)s[hi - 1].v) : 0.0) * cf;
    }
    double cb = 0.0;
    for (int t = T - 1; t >= 0; --t) {
      const int64_t lo = (int64_t)t * ch, hi = lo + ch < n ? lo + ch : n;
      carry_b[(size_t)t * m + c] = cb;
      if (lo < hi) cb = fold_b[(size_t)t * m + c] + (hi < n ? exp((double)s[lo].v - (double)s[hi].v) : 0.0) * cb;
    }
  }
  /* pass 2: both recurrences from the carries; y = L + U - x */
#pragma omp parallel for num_threads(T) schedule(static, 1)
  for (int t = 0; t < T; ++t) {
    const int64_t lo = (int64_t)t * ch, hi = lo + ch < n ? lo + ch : n;
    for (int64_t c = 0; c < m; ++c) {
      double l = carry_f[(size_t)t * m + c];
      for (int64_t i = lo; i < hi; ++i) {
        l = (double)x[(size_t)s[i].i * m + c] + (i > 0 ? exp((double)s[i - 1].v - (double)s[i].v) : 0.0) * l;
        L[(size_t)i * m + c] = l;
      }
      double u = carry_b[(size_t)t * m + c];
      for (int64_t i = hi - 1; i >= lo; --i) {
        const double xv = (double)x[(size_t)s[i].i * m + c];
        u = xv + (i + 1 < n ? exp((double)s[i].v - (double)s[i + 1].v) : 0.0) * u;
        y[(size_t)s[i].i * m + c] = L[(size_t)i * m + c] + u - xv;
      }
    }
  }
  free(s);
  free(L);
  free(agg);
  return 0;
}
