/*
 * LAPLEX CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, sequential, float64 implementation of the LAPLEX operator apply
 *     y_i = sum_j exp(-|a_i - b_j|) * x_j                      (optionally * cos(phi_i - psi_j))
 * following the exact scan algebra of "LAPLEX: The FFT of Learnable Laplace
 * Kernels" (gist.science technical summary, section 2.1 "The Operator" and
 * section 2.2 "Exact Scan Algebra").  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the GPU library shares
 * no code with it.
 *
 * Conventions (where the pages are silent):
 *  - sort: ascending, stable (equal anchors keep their input order), -0.0 and
 *    +0.0 compare equal, NaN/Inf anchors are rejected (return -1);
 *  - general case: an input anchor b_j equal to an output anchor a_i counts
 *    on the "left" side (b_j <= a_i); the weight is exp(0) = 1 either way;
 *  - matrices are row-major, x is (rows x m), y is (rows x m) float64.
 *
 * Parity: pinned by the closed-form and invariant checks of the oracle
 * test-suite (Kac-Murdock-Szego inverse, tridiagonal inverse of the Markov
 * exponential covariance, Toeplitz/FFT reduction, symmetry/adjointness,
 * K e_j = column j, zero-temperature permutation limit, geometric row sums).
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  float v;
  uint32_t i;
} vi_t;

/* bottom-up merge of two sorted runs; takes from the left run on equality
 * (this is what makes the sort stable) */
static void merge_runs(const vi_t* src, vi_t* dst, int64_t lo, int64_t mid, int64_t hi) {
  int64_t p = lo, q = mid, o = lo;
  while (p < mid && q < hi) {
    if (src[q].v < src[p].v)
      dst[o++] = src[q++];
    else
      dst[o++] = src[p++];
  }
  while (p < mid) dst[o++] = src[p++];
  while (q < hi) dst[o++] = src[q++];
}

/* Sort of the anchors ("after sorting the anchors", section 2.2, symmetric
 * case).  perm[r] = input index of the r-th smallest anchor.  Returns 0, or
 * -1 when an anchor is not finite, or -2 when out of memory. */
int lo_stable_argsort(const float* a, int64_t n, uint32_t* perm) {
  if (n <= 0) return 0;
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return -1;
  vi_t* buf0 = (vi_t*)malloc(sizeof(vi_t) * (size_t)n);
  vi_t* buf1 = (vi_t*)malloc(sizeof(vi_t) * (size_t)n);
  if (!buf0 || !buf1) {
    free(buf0);
    free(buf1);
    return -2;
  }
  for (int64_t i = 0; i < n; ++i) {
    buf0[i].v = a[i];
    buf0[i].i = (uint32_t)i;
  }
  /* short runs by insertion sort (stable: shifts only strictly greater) */
  const int64_t RUN = 32;
  for (int64_t lo = 0; lo < n; lo += RUN) {
    int64_t hi = lo + RUN < n ? lo + RUN : n;
    for (int64_t i = lo + 1; i < hi; ++i) {
      vi_t t = buf0[i];
      int64_t j = i - 1;
      while (j >= lo && buf0[j].v > t.v) {
        buf0[j + 1] = buf0[j];
        --j;
      }
      buf0[j + 1] = t;
    }
  }
  vi_t *src = buf0, *dst = buf1;
  for (int64_t w = RUN; w < n; w *= 2) {
    for (int64_t lo = 0; lo < n; lo += 2 * w) {
      int64_t mid = lo + w < n ? lo + w : n;
      int64_t hi = lo + 2 * w < n ? lo + 2 * w : n;
      merge_runs(src, dst, lo, mid, hi);
    }
    vi_t* t = src;
    src = dst;
    dst = t;
  }
  for (int64_t i = 0; i < n; ++i) perm[i] = src[i].i;
  free(buf0);
  free(buf1);
  return 0;
}

/* Symmetric case a = b (section 2.2): after sorting, K = lower + upper - diag.
 * Lower part: L_0 = x_0, L_i = x_i + exp(a_{i-1} - a_i) L_{i-1}  (prefix scan);
 * upper part: U_{n-1} = x_{n-1}, U_i = x_i + exp(a_i - a_{i+1}) U_{i+1}
 * (suffix scan); y[perm[i]] = L_i + U_i - x_i. */
int lo_sym_apply(const float* a, int64_t n, int64_t m, const float* x, double* y) {
  if (n <= 0 || m <= 0) return 0;
  uint32_t* perm = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)n);
  double* as = (double*)malloc(sizeof(double) * (size_t)n);
  double* ls = (double*)malloc(sizeof(double) * (size_t)n * (size_t)m);
  double* u = (double*)malloc(sizeof(double) * (size_t)m);
  int rc = (perm && as && ls && u) ? 0 : -2;
  if (rc == 0) rc = lo_stable_argsort(a, n, perm);
  if (rc == 0) {
    for (int64_t i = 0; i < n; ++i) as[i] = (double)a[perm[i]];
    /* lower-triangular (prefix) recurrence */
    for (int64_t c = 0; c < m; ++c) ls[c] = (double)x[(size_t)perm[0] * m + c];
    for (int64_t i = 1; i < n; ++i) {
      double d = exp(as[i - 1] - as[i]);
      const float* xr = x + (size_t)perm[i] * m;
      for (int64_t c = 0; c < m; ++c) ls[i * m + c] = (double)xr[c] + d * ls[(i - 1) * m + c];
    }
    /* upper-triangular (suffix) recurrence, combined on the fly; nothing
     * follows the last element, so the carry into it is zero */
    for (int64_t c = 0; c < m; ++c) u[c] = 0.0;
    for (int64_t i = n - 1; i >= 0; --i) {
      const float* xr = x + (size_t)perm[i] * m;
      double d = (i == n - 1) ? 0.0 : exp(as[i] - as[i + 1]);
      double* yr = y + (size_t)perm[i] * m;
      for (int64_t c = 0; c < m; ++c) {
        u[c] = (double)xr[c] + d * u[c];
        yr[c] = ls[i * m + c] + u[c] - (double)xr[c];
      }
    }
  }
  free(perm);
  free(as);
  free(ls);
  free(u);
  return rc;
}

/* first index p with as[p] >= v (number of sorted anchors strictly below v) */
static int64_t lower_bound_d(const double* as, int64_t n, double v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (as[mid] < v)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

/* General case a != b (section 2.2): each input anchor b_j falls into the
 * interval (a_{p-1}, a_p] of the sorted output anchors, p = #{a < b_j}.  Its
 * contribution is summarised at the interval's right end in u (for outputs at
 * or above b_j) and at its left end in v (for outputs below b_j):
 *     u_p     += exp(b_j - a_p)     x_j        (p <= n-1)
 *     v_{p-1} += exp(a_{p-1} - b_j) x_j        (p >= 1)
 * and the symmetric scan primitive propagates them:
 *     Y_i = u_i + exp(a_{i-1} - a_i) Y_{i-1},   Z_i = v_i + exp(a_i - a_{i+1}) Z_{i+1},
 *     y[perm_a[i]] = Y_i + Z_i   (no diagonal term). */
int lo_general_apply(const float* a, int64_t n, const float* b, int64_t k, int64_t m, const float* x, double* y) {
  if (n <= 0 || m <= 0) return 0;
  if (k <= 0) {
    memset(y, 0, sizeof(double) * (size_t)n * (size_t)m);
    return 0;
  }
  uint32_t* pa = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)n);
  uint32_t* pb = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)k);
  double* as = (double*)malloc(sizeof(double) * (size_t)n);
  double* uu = (double*)calloc((size_t)n * (size_t)m, sizeof(double));
  double* vv = (double*)calloc((size_t)n * (size_t)m, sizeof(double));
  double* z = (double*)malloc(sizeof(double) * (size_t)m);
  int rc = (pa && pb && as && uu && vv && z) ? 0 : -2;
  if (rc == 0) rc = lo_stable_argsort(a, n, pa);
  if (rc == 0) rc = lo_stable_argsort(b, k, pb);
  if (rc == 0) {
    for (int64_t i = 0; i < n; ++i) as[i] = (double)a[pa[i]];
    for (int64_t j = 0; j < k; ++j) {
      double bj = (double)b[pb[j]];
      const float* xr = x + (size_t)pb[j] * m;
      int64_t p = lower_bound_d(as, n, bj);
      if (p < n) {
        double w = exp(bj - as[p]);
        for (int64_t c = 0; c < m; ++c) uu[p * m + c] += w * (double)xr[c];
      }
      if (p >= 1) {
        double w = exp(as[p - 1] - bj);
        for (int64_t c = 0; c < m; ++c) vv[(p - 1) * m + c] += w * (double)xr[c];
      }
    }
    /* forward scan of u in place */
    for (int64_t i = 1; i < n; ++i) {
      double d = exp(as[i - 1] - as[i]);
      for (int64_t c = 0; c < m; ++c) uu[i * m + c] += d * uu[(i - 1) * m + c];
    }
    /* backward scan of v, combined */
    for (int64_t c = 0; c < m; ++c) z[c] = 0.0;
    for (int64_t i = n - 1; i >= 0; --i) {
      double d = (i == n - 1) ? 0.0 : exp(as[i] - as[i + 1]);
      double* yr = y + (size_t)pa[i] * m;
      for (int64_t c = 0; c < m; ++c) {
        z[c] = vv[i * m + c] + d * z[c];
        yr[c] = uu[i * m + c] + z[c];
      }
    }
  }
  free(pa);
  free(pb);
  free(as);
  free(uu);
  free(vv);
  free(z);
  return rc;
}

/* Phased operator (section 2.1): K_ij = exp(-|a_i - b_j|) cos(phi_i - psi_j).
 * Written with complex numbers: cos(phi_i - psi_j) = Re(e^{i phi_i} e^{-i psi_j}),
 * so y = Re(e^{i phi} .* K0 (e^{-i psi} .* x)) where K0 is the unphased operator,
 * evaluated with the same scans as above in complex arithmetic.
 * b == NULL selects the symmetric operator (b = a, psi = phi, k = n). */
int lo_phased_apply(const float* a, const float* phi, int64_t n, const float* b, const float* psi, int64_t k,
                    int64_t m, const float* x, double* y) {
  if (n <= 0 || m <= 0) return 0;
  int sym = (b == NULL);
  if (sym) {
    b = a;
    psi = phi;
    k = n;
  }
  if (k <= 0) {
    memset(y, 0, sizeof(double) * (size_t)n * (size_t)m);
    return 0;
  }
  uint32_t* pa = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)n);
  uint32_t* pb = sym ? pa : (uint32_t*)malloc(sizeof(uint32_t) * (size_t)k);
  double* as = (double*)malloc(sizeof(double) * (size_t)n);
  double complex* uu = (double complex*)calloc((size_t)n * (size_t)m, sizeof(double complex));
  double complex* vv = (double complex*)calloc((size_t)n * (size_t)m, sizeof(double complex));
  double complex* z = (double complex*)malloc(sizeof(double complex) * (size_t)m);
  int rc = (pa && pb && as && uu && vv && z) ? 0 : -2;
  if (rc == 0) rc = lo_stable_argsort(a, n, pa);
  if (rc == 0 && !sym) rc = lo_stable_argsort(b, k, pb);
  if (rc == 0) {
    for (int64_t i = 0; i < n; ++i) as[i] = (double)a[pa[i]];
    if (sym) {
      /* symmetric: inject z_j = e^{-i phi_j} x_j at its own sorted position
       * into both directions; the diagonal is removed at the end */
      for (int64_t i = 0; i < n; ++i) {
        double ph = (double)phi[pa[i]];
        double complex e = cexp(-I * ph);
        const float* xr = x + (size_t)pa[i] * m;
        for (int64_t c = 0; c < m; ++c) {
          uu[i * m + c] = e * (double)xr[c];
          vv[i * m + c] = e * (double)xr[c];
        }
      }
    } else {
      for (int64_t j = 0; j < k; ++j) {
        double bj = (double)b[pb[j]];
        double complex e = cexp(-I * (double)psi[pb[j]]);
        const float* xr = x + (size_t)pb[j] * m;
        int64_t p = lower_bound_d(as, n, bj);
        if (p < n) {
          double w = exp(bj - as[p]);
          for (int64_t c = 0; c < m; ++c) uu[p * m + c] += w * e * (double)xr[c];
        }
        if (p >= 1) {
          double w = exp(as[p - 1] - bj);
          for (int64_t c = 0; c < m; ++c) vv[(p - 1) * m + c] += w * e * (double)xr[c];
        }
      }
    }
    for (int64_t i = 1; i < n; ++i) {
      double d = exp(as[i - 1] - as[i]);
      for (int64_t c = 0; c < m; ++c) uu[i * m + c] += d * uu[(i - 1) * m + c];
    }
    for (int64_t c = 0; c < m; ++c) z[c] = 0.0;
    for (int64_t i = n - 1; i >= 0; --i) {
      double d = (i == n - 1) ? 0.0 : exp(as[i] - as[i + 1]);
      double complex eo = cexp(I * (double)phi[pa[i]]);
      const float* xr = x + (size_t)pa[i] * m;
      double* yr = y + (size_t)pa[i] * m;
      for (int64_t c = 0; c < m; ++c) {
        z[c] = vv[i * m + c] + d * z[c];
        double complex w = uu[i * m + c] + z[c];
        /* symmetric: the diagonal entry exp(0) cos(0) x_i was injected twice */
        if (sym) w -= cexp(-I * (double)phi[pa[i]]) * (double)xr[c];
        yr[c] = creal(eo * w);
      }
    }
  }
  free(pa);
  if (!sym) free(pb);
  free(as);
  free(uu);
  free(vv);
  free(z);
  return rc;
}

/* Selected rows of the operator by its plain definition (section 2.1), for
 * spot checks of inputs too large for a full dense product:
 *   y[r][c]   = sum_j exp(-|a[rows[r]] - b_j|) cos(phi - psi) x[j][c]
 *   env[r][c] = sum_j exp(-|a[rows[r]] - b_j|) |x[j][c]|
 * (phi/psi NULL: unphased).  Terms with |a - b| >= 746 are skipped: their
 * weight exp(-|a - b|) underflows to exactly 0 in float64, so the sums are
 * unchanged.  One pass over b for all rows. */
int lo_dense_rows(const float* a, const float* phi, const int64_t* rows, int64_t nrows, const float* b, const float* psi,
                  int64_t k, int64_t m, const float* x, double* y, double* env) {
  if (nrows <= 0 || m <= 0) return 0;
  double* ai = (double*)malloc(sizeof(double) * (size_t)nrows);
  double* pi = (double*)malloc(sizeof(double) * (size_t)nrows);
  if (!ai || !pi) {
    free(ai);
    free(pi);
    return -2;
  }
  for (int64_t r = 0; r < nrows; ++r) {
    ai[r] = (double)a[rows[r]];
    pi[r] = phi ? (double)phi[rows[r]] : 0.0;
  }
  memset(y, 0, sizeof(double) * (size_t)(nrows * m));
  memset(env, 0, sizeof(double) * (size_t)(nrows * m));
  for (int64_t j = 0; j < k; ++j) {
    const double bj = (double)b[j];
    const float* xr = x + (size_t)j * m;
    for (int64_t r = 0; r < nrows; ++r) {
      const double d = fabs(ai[r] - bj);
      if (d >= 746.0) continue;
      const double w = exp(-d);
      const double wc = phi ? w * cos(pi[r] - (double)psi[j]) : w;
      for (int64_t c = 0; c < m; ++c) {
        y[r * m + c] += wc * (double)xr[c];
        env[r * m + c] += w * fabs((double)xr[c]);
      }
    }
  }
  free(ai);
  free(pi);
  return 0;
}

/* ------------------------------------------------------------------ backward
 * The operator is differentiable in its anchors (technical summary, section
 * 2.3, expressivity and limits: the relation to the FFT keeps exactness and
 * differentiability with respect to the anchors).  With y = K x and an upstream gradient g = dL/dy, the chain rule
 * on K_ij = exp(-|a_i - b_j|) gives
 *     dL/dx   = K^T g
 *     dL/da_i = - sum_c g_ic  S_{b,x_c}(a_i),   S_{s,v}(t) = sum_j sign(t - s_j) exp(-|t - s_j|) v_j
 *     dL/db_j = - sum_c x_jc  S_{a,g_c}(b_j)
 * and in the symmetric case (b = a, one anchor set) both terms land on a:
 *     dL/da_i = - sum_c [ g_ic S_{a,x_c}(a_i) + x_ic S_{a,g_c}(a_i) ].
 * sign(0) = 0: equal anchors contribute nothing, the value a central
 * difference gives at a tie (|t| has a kink there).
 *
 * S is evaluated from the sorted sources: with the stable prefix and suffix
 * scans  P_t = sum_{j<=t} exp(s_j - s_t) v_j  and  Q_t = sum_{j>=t} exp(s_t - s_j) v_j,
 *     S(t) = exp(s_{p-1} - t) P_{p-1} - exp(t - s_q) Q_q,
 * p = #{s_j < t} (lower bound), q = #{s_j <= t} (upper bound); every factor
 * is a single exp of a non-positive difference. */

/* number of sorted anchors <= v */
static int64_t upper_bound_d(const double* as, int64_t n, double v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (as[mid] <= v)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

/* out[e*m + c] = S_{s, v_c}(t_e) for sources s (ns, unsorted) with values v
 * (ns x m, row-major) and evaluation points t (ne). */
static int signed_sums(const float* s, int64_t ns, const float* v, int64_t m, const float* t, int64_t ne, double* out) {
  if (ne <= 0 || m <= 0) return 0;
  if (ns <= 0) {
    memset(out, 0, sizeof(double) * (size_t)ne * (size_t)m);
    return 0;
  }
  uint32_t* ps = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)ns);
  double* ss = (double*)malloc(sizeof(double) * (size_t)ns);
  double* P = (double*)malloc(sizeof(double) * (size_t)ns * (size_t)m);
  double* Q = (double*)malloc(sizeof(double) * (size_t)ns * (size_t)m);
  int rc = (ps && ss && P && Q) ? 0 : -2;
  if (rc == 0) rc = lo_stable_argsort(s, ns, ps);
  if (rc == 0) {
    for (int64_t j = 0; j < ns; ++j) ss[j] = (double)s[ps[j]];
    for (int64_t c = 0; c < m; ++c) P[c] = (double)v[(size_t)ps[0] * m + c];
    for (int64_t j = 1; j < ns; ++j) {
      const double d = exp(ss[j - 1] - ss[j]);
      for (int64_t c = 0; c < m; ++c) P[j * m + c] = (double)v[(size_t)ps[j] * m + c] + d * P[(j - 1) * m + c];
    }
    for (int64_t c = 0; c < m; ++c) Q[(ns - 1) * m + c] = (double)v[(size_t)ps[ns - 1] * m + c];
    for (int64_t j = ns - 2; j >= 0; --j) {
      const double d = exp(ss[j] - ss[j + 1]);
      for (int64_t c = 0; c < m; ++c) Q[j * m + c] = (double)v[(size_t)ps[j] * m + c] + d * Q[(j + 1) * m + c];
    }
    for (int64_t e = 0; e < ne; ++e) {
      const double te = (double)t[e];
      const int64_t p = lower_bound_d(ss, ns, te), q = upper_bound_d(ss, ns, te);
      const double wl = p >= 1 ? exp(ss[p - 1] - te) : 0.0;
      const double wu = q < ns ? exp(te - ss[q]) : 0.0;
      for (int64_t c = 0; c < m; ++c) {
        const double lo = p >= 1 ? wl * P[(p - 1) * m + c] : 0.0;
        const double hi = q < ns ? wu * Q[q * m + c] : 0.0;
        out[e * m + c] = lo - hi;
      }
    }
  }
  free(ps);
  free(ss);
  free(P);
  free(Q);
  return rc;
}

/* Symmetric backward: dx = K g (n x m), da (n). */
int lo_sym_backward(const float* a, int64_t n, int64_t m, const float* x, const float* g, double* dx, double* da) {
  if (n <= 0 || m <= 0) return 0;
  int rc = lo_sym_apply(a, n, m, g, dx);
  if (rc != 0) return rc;
  double* sx = (double*)malloc(sizeof(double) * (size_t)n * (size_t)m);
  double* sg = (double*)malloc(sizeof(double) * (size_t)n * (size_t)m);
  rc = (sx && sg) ? 0 : -2;
  if (rc == 0) rc = signed_sums(a, n, x, m, a, n, sx);
  if (rc == 0) rc = signed_sums(a, n, g, m, a, n, sg);
  if (rc == 0) {
    for (int64_t i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int64_t c = 0; c < m; ++c)
        acc += (double)g[i * m + c] * sx[i * m + c] + (double)x[i * m + c] * sg[i * m + c];
      da[i] = -acc;
    }
  }
  free(sx);
  free(sg);
  return rc;
}

/* General backward (K is n x k, rows a, columns b): dx = K^T g (k x m),
 * da (n), db (k). */
int lo_general_backward(const float* a, int64_t n, const float* b, int64_t k, int64_t m, const float* x, const float* g,
                        double* dx, double* da, double* db) {
  if (m <= 0) return 0;
  if (k > 0) {
    int rc0 = lo_general_apply(b, k, a, n, m, g, dx);
    if (rc0 != 0) return rc0;
  }
  double* sa = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)m);
  double* sb = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1) * (size_t)m);
  int rc = (sa && sb) ? 0 : -2;
  if (rc == 0) rc = signed_sums(b, k, x, m, a, n, sa);
  if (rc == 0) rc = signed_sums(a, n, g, m, b, k, sb);
  if (rc == 0) {
    for (int64_t i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int64_t c = 0; c < m; ++c) acc += (double)g[i * m + c] * sa[i * m + c];
      da[i] = -acc;
    }
    for (int64_t j = 0; j < k; ++j) {
      double acc = 0.0;
      for (int64_t c = 0; c < m; ++c) acc += (double)x[j * m + c] * sb[j * m + c];
      db[j] = -acc;
    }
  }
  free(sa);
  free(sb);
  return rc;
}

/* Anchor gradient of the symmetric backward at selected rows, by the plain
 * definition (no sort), and its envelope
 *     env_r = sum_c sum_j exp(-|a_i - a_j|) (|g_ic| |x_jc| + |x_ic| |g_jc|),   i = rows[r],
 * for sizes where only spot rows can be checked.  Terms with |a_i - a_j| >= 746
 * are skipped (exp underflows to 0 in float64). */
int lo_backward_rows(const float* a, int64_t n, int64_t m, const float* x, const float* g, const int64_t* rows, int64_t nrows,
                     double* da, double* env) {
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = rows[r];
    if (i < 0 || i >= n) return -3;
    const double ai = (double)a[i];
    double acc = 0.0, e = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      const double d = ai - (double)a[j];
      const double ad = fabs(d);
      if (ad >= 746.0) continue;
      const double w = exp(-ad);
      const double sg = d > 0.0 ? 1.0 : (d < 0.0 ? -1.0 : 0.0);
      for (int64_t c = 0; c < m; ++c) {
        const double gi = (double)g[i * m + c], xi = (double)x[i * m + c];
        const double xj = (double)x[j * m + c], gj = (double)g[j * m + c];
        acc += sg * w * (gi * xj + xi * gj);
        e += w * (fabs(gi) * fabs(xj) + fabs(xi) * fabs(gj));
      }
    }
    da[r] = -acc;
    env[r] = e;
  }
  return 0;
}
