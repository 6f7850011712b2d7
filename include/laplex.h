/*
 * laplex.h -- C interface of the LAPLEX operator library for AMD Instinct
 * MI355X (gfx950).
 *
 * The operator ("LAPLEX: The FFT of Learnable Laplace Kernels", technical
 * summary, section 2.1 "The Operator"):
 *
 *     LAPLEX(a, b)_ij           = exp(-|a_i - b_j|)                  a in R^n, b in R^k
 *     LAPLEX(a, phi; b, psi)_ij = exp(-|a_i - b_j|) cos(phi_i - psi_j)
 *
 * applied to a block of m right-hand sides, y = LAPLEX x, in O((n + k) log)
 * work through the sort and prefix/suffix scan algebra of section 2.2
 * ("Exact Scan Algebra"); the dense matrix is never formed.  Row index i is
 * the output (anchors a), column index j the input (anchors b).
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller (for example
 *    the data of torch tensors).  float arrays are IEEE binary32; permutations
 *    are uint32.  All must be 4-byte aligned.
 *  - x is row-major (rows x m): row r holds the m columns of input r
 *    contiguously; y likewise (n x m).  x, y, phi and psi are in the ORIGINAL
 *    (unsorted) order of their anchors.
 *  - Work is enqueued on `stream` and is asynchronous: argument errors are
 *    returned synchronously, nothing is waited on.  The library allocates no
 *    device memory and keeps no global state (apart from the opt-in launch
 *    profiler at the end of this header); each call needs its own workspace
 *    of at least laplex_workspace_bytes(...) bytes (256-byte aligned), and
 *    calls whose workspaces differ may run concurrently on different streams.
 *  - Outputs must not overlap inputs or the workspace.
 *  - n, k < 2^32 (permutations are uint32).  n == 0 or m == 0 is a no-op.
 */
#ifndef LAPLEX_H
#define LAPLEX_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LAPLEX_OK = 0,
  LAPLEX_ERR_NULL = 1,       /* a required pointer is NULL */
  LAPLEX_ERR_SIZE = 2,       /* n or k >= 2^32, or m too large */
  LAPLEX_ERR_ALIGN = 3,      /* a pointer is not 4-byte aligned (workspace: 256-byte) */
  LAPLEX_ERR_WORKSPACE = 4,  /* ws_bytes smaller than laplex_workspace_bytes(...) */
  LAPLEX_ERR_NONFINITE = 5,  /* an anchor was NaN or +-Inf (reported by laplex_status_poll) */
  LAPLEX_ERR_HIP = 6,        /* a HIP launch or runtime call failed */
  LAPLEX_ERR_OVERLAP = 7,    /* an output overlaps an input or the workspace */
  LAPLEX_ERR_STALLED = 8,    /* a look-back wait hit its spin limit (reported by laplex_status_poll) */
  LAPLEX_ERR_ARG = 9,        /* any other invalid argument */
  LAPLEX_ERR_SCRATCH = 10    /* the call needs more than LAPLEX_SCRATCH_BYTES of static scratch */
} laplex_status;

/* Operations, for laplex_workspace_bytes. */
enum {
  LAPLEX_OP_SORT = 0,
  LAPLEX_OP_SYM = 1,
  LAPLEX_OP_GENERAL = 2,
  LAPLEX_OP_PHASED = 3,         /* symmetric phased operator (b = a, psi = phi) */
  LAPLEX_OP_PHASED_GENERAL = 4, /* phased operator with a != b */
  LAPLEX_OP_SYM_BACKWARD = 5,   /* backward of the symmetric operator */
  LAPLEX_OP_GENERAL_BACKWARD = 6, /* backward of the general operator */
  LAPLEX_OP_GRAM = 7,             /* weighted Gram matrix */
  LAPLEX_OP_PHASED_BACKWARD = 8,  /* backward of the symmetric phased operator */
  LAPLEX_OP_PHASED_GENERAL_BACKWARD = 9, /* backward of the phased operator with a != b */
  LAPLEX_OP_SORT_SYM = 10,               /* sort and symmetric operator in one call */
  LAPLEX_OP_SORT_GENERAL = 11            /* sort of b and general operator in one call */
};

/* Bytes of workspace one call of `op` needs for n output anchors, k input
 * anchors (ignored by the symmetric operations) and m columns.  Returns 0 when
 * the sizes are out of range. */
size_t laplex_workspace_bytes(int op, uint64_t n, uint64_t k, uint32_t m);

/* Bytes of the optional sort route for n anchors (see laplex_sort_anchors);
 * 0 when n is out of range. */
size_t laplex_route_bytes(uint64_t n);

/* Sort of the anchors ("after sorting the anchors", section 2.2, symmetric
 * case): perm[r] is the input index of the r-th smallest anchor and
 * a_sorted[r] = a[perm[r]] bit for bit.  The order is ascending and stable
 * (equal anchors keep their input order; -0.0 and +0.0 count as equal).
 * The triple (a_sorted, perm, route) is the sort handle every apply takes, so
 * one sort serves any number of applies.  NaN/Inf anchors leave the outputs
 * undefined and raise LAPLEX_ERR_NONFINITE in laplex_status_poll(ws).
 * a: n floats (input); a_sorted: n floats (output); perm: n uint32 (output);
 * route: NULL, or a device buffer of laplex_route_bytes(n) bytes (256-byte
 * aligned, output) that records, for each of the four radix passes, where
 * every element went; an apply given the route moves x into sorted order and
 * y back along it with coalesced passes instead of per-element gathers and
 * scatters through perm (used when m <= 4; the results are bitwise the same);
 * ws: workspace of laplex_workspace_bytes(LAPLEX_OP_SORT, n, 0, 1) bytes. */
laplex_status laplex_sort_anchors(const float* a, uint64_t n, float* a_sorted, uint32_t* perm, void* route, size_t route_bytes,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Waits for `stream`, then returns the sticky device-side status of the last
 * sort that used `ws` (LAPLEX_OK, LAPLEX_ERR_NONFINITE or LAPLEX_ERR_STALLED).
 * A look-back wait that reaches its spin limit gives up: the watchdog flag is
 * raised, the remaining passes stop at once, every kernel exits, and the
 * sort's outputs are undefined.  For failure-path tests,
 * LAPLEX_DEBUG_STALL=<k> in the environment makes laplex_sort_anchors (only
 * this entry point) run its look-back passes without publishing and with a
 * spin limit of k, which forces that path. */
laplex_status laplex_status_poll(const void* ws, hipStream_t stream);

/* Symmetric operator y = LAPLEX(a, a) x (section 2.2, symmetric case: lower
 * part by a prefix scan y_i = x_i + exp(a_{i-1} - a_i) y_{i-1}, upper part by
 * the mirrored suffix scan, combined as lower + upper - diagonal).
 * a_sorted, perm, route: the sort handle of a (n each; route may be NULL);
 * x: n x m (input, original order); y: n x m (output, original order);
 * ws: laplex_workspace_bytes(LAPLEX_OP_SYM, n, 0, m) bytes. */
laplex_status laplex_matvec_sym(const float* a_sorted, const uint32_t* perm, const void* route, uint64_t n, uint32_t m,
                                const float* x, float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* laplex_matvec_sym without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is the library's static
 * device scratch array of LAPLEX_SCRATCH_BYTES, one per GPU, held from the
 * first call on that GPU until the process ends; its device address is
 * looked up once per GPU (hipGetSymbolAddress, on the stream's device) and
 * the call allocates nothing.  Arguments, layout and results as
 * laplex_matvec_sym (bitwise the same output).  The call fits when
 * laplex_workspace_bytes(LAPLEX_OP_SYM, n, 0, m) <= LAPLEX_SCRATCH_BYTES
 * (e.g. n * m up to about 4 * 2^20 with a route); larger calls return
 * LAPLEX_ERR_SCRATCH before launching anything.  Every call on one GPU uses
 * the same scratch and keeps nothing from the last call in it: calls that
 * overlap in time on one GPU (different streams, or host threads) race and
 * must be serialised by the caller. */
#define LAPLEX_SCRATCH_BYTES (64ull << 20)
laplex_status laplex_matvec_sym_noalloc(const float* a_sorted, const uint32_t* perm, const void* route, uint64_t n, uint32_t m,
                                        const float* x, float* y, hipStream_t stream);

/* The symmetric operator from unsorted anchors in one call: the sort of
 * laplex_sort_anchors followed by laplex_matvec_sym (section 2.2, symmetric
 * case: sort, then the two scans), for callers that apply K(a) once.  With
 * m == 1 the inputs ride through the sort's passes as the keys' values (no
 * permutation is formed and x is not moved separately); otherwise the sort
 * handle is built inside the workspace and the apply takes it.  The result
 * is bitwise the same as laplex_sort_anchors + laplex_matvec_sym with a route.
 * a: n floats; x: n x m (inputs, original order); y: n x m (output, original
 * order, must not overlap a, x or ws); ws: laplex_workspace_bytes(
 * LAPLEX_OP_SORT_SYM, n, 0, m) bytes; it holds the sort workspace, so
 * laplex_status_poll(ws) reports non-finite anchors and stalls as for a sort. */
laplex_status laplex_sort_matvec_sym(const float* a, uint64_t n, uint32_t m, const float* x, float* y, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* The general operator y = LAPLEX(a, b) x from unsorted anchors in one call
 * (section 2.2, general case), for few input anchors: only b is sorted.  The
 * two scans run over sorted b, Fi_j = sum_{j' <= j} exp(-(b_j - b_j')) x_j'
 * and U_j = sum_{j' >= j} exp(-(b_j' - b_j)) x_j', and each output anchor a_i
 * finds p = #{b_j <= a_i} by binary search (b before a on ties, as in
 * laplex_matvec_general) and takes y_i = exp(-(a_i - b_{p-1})) Fi_{p-1} +
 * exp(-(b_p - a_i)) U_p.  The same sum split at the same place as the merged
 * scan, with no sort of a: O(k log k + n log k).  Best while b and the two
 * scans fit in the caches (k up to about 2^18 at m = 1); otherwise sort both
 * and use laplex_matvec_general.  The result equals laplex_matvec_general's
 * within rounding (not bitwise).
 * a: n floats; b: k floats; x: k x m (original order of b); y: n x m (output,
 * original order of a; must not overlap a, b, x or ws); k == 0 gives y = 0;
 * ws: laplex_workspace_bytes(LAPLEX_OP_SORT_GENERAL, n, k, m) bytes (it holds
 * b's sort workspace: laplex_status_poll(ws) reports non-finite a or b). */
laplex_status laplex_sort_matvec_general(const float* a, uint64_t n, const float* b, uint64_t k, uint32_t m, const float* x,
                                         float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of laplex_sort_matvec_sym from what that call left in its
 * workspace (the sorted anchors, the route or permutation, and x in sorted
 * order): dx = K g and the anchor gradient da (section 2.3: the operator is
 * differentiable in its anchors; da_i = -sum_j sign(a_i - a_j) K_ij
 * sum_c (g_ic x_jc + x_ic g_jc), ties contributing nothing), as
 * laplex_backward_sym computes them.  Only g is moved into sorted order.
 * fwd_ws: the workspace of a laplex_sort_matvec_sym call with the same a, x, n
 * and m, unchanged since (fwd_ws_bytes as passed to it); g: n x m (input,
 * original order); dx: n x m, da: n (outputs, original order); ws:
 * laplex_workspace_bytes(LAPLEX_OP_SYM_BACKWARD, n, 0, m) bytes, not
 * overlapping fwd_ws. */
laplex_status laplex_sort_matvec_sym_backward(const void* fwd_ws, size_t fwd_ws_bytes, uint64_t n, uint32_t m, const float* g,
                                              float* dx, float* da, void* ws, size_t ws_bytes, hipStream_t stream);

/* General operator y = LAPLEX(a, b) x with a != b (section 2.2, general case:
 * the input anchors b are placed into the intervals of the sorted output
 * anchors a and propagated with the same scan primitive; here the two sorted
 * sequences are merged, b before a on equal anchors, and scanned once in
 * each direction).  A b anchor equal to an a anchor couples with weight 1.
 * a_sorted, perm_a, route_a: sort handle of a (n); b_sorted, perm_b, route_b:
 * sort handle of b (k); either route may be NULL; x: k x m (input);
 * y: n x m (output); ws: laplex_workspace_bytes(LAPLEX_OP_GENERAL, n, k, m)
 * bytes.  k == 0 sets y to zero. */
laplex_status laplex_matvec_general(const float* a_sorted, const uint32_t* perm_a, const void* route_a, uint64_t n,
                                    const float* b_sorted, const uint32_t* perm_b, const void* route_b, uint64_t k, uint32_t m,
                                    const float* x, float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Phased operator y = LAPLEX(a, phi; b, psi) x (section 2.1, phased
 * extension), computed as two real scans of the columns cos(psi) x and
 * sin(psi) x, recombined with cos(phi) and sin(phi)
 * (cos(phi_i - psi_j) = cos phi_i cos psi_j + sin phi_i sin psi_j).
 * b_sorted == NULL selects the symmetric operator b = a, psi = phi (perm_b,
 * route_b, psi and k are then ignored and x is n x m).  phi: n floats, psi:
 * k floats, both in original order; routes may be NULL.
 * ws: laplex_workspace_bytes(LAPLEX_OP_PHASED or LAPLEX_OP_PHASED_GENERAL, n, k, m). */
laplex_status laplex_matvec_phased(const float* a_sorted, const uint32_t* perm_a, const void* route_a, const float* phi,
                                   uint64_t n, const float* b_sorted, const uint32_t* perm_b, const void* route_b,
                                   const float* psi, uint64_t k, uint32_t m, const float* x, float* y, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Backward of the symmetric operator y = LAPLEX(a, a) x.  The operator is
 * differentiable in its anchors (technical summary, section 2.3, relation to
 * the FFT); for an upstream gradient g = dL/dy the chain rule on
 * exp(-|a_i - a_j|) gives
 *     dx   = LAPLEX(a, a) g                                        (n x m)
 *     da_i = - sum_c [ g_ic S(x_c)_i + x_ic S(g_c)_i ]             (n)
 *     S(v)_i = sum_j sign(a_i - a_j) exp(-|a_i - a_j|) v_j,  sign(0) = 0,
 * so tied anchors contribute nothing to each other's gradient (the value a
 * central difference gives at the kink of |t|).  S is computed with the same
 * prefix/suffix scans, once with the kernel's decay and once summing over
 * tied anchors only.
 * a_sorted, perm, route: the sort handle of a (route may be NULL);
 * x, g: n x m (inputs, original order); dx: n x m and da: n (outputs,
 * original order); ws: laplex_workspace_bytes(LAPLEX_OP_SYM_BACKWARD, n, 0, m). */
laplex_status laplex_backward_sym(const float* a_sorted, const uint32_t* perm, const void* route, uint64_t n, uint32_t m,
                                  const float* x, const float* g, float* dx, float* da, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* Backward of the symmetric phased operator y = LAPLEX(a, phi; a, phi) x
 * (technical summary, section 2.1, phased extension; anchors and phases are
 * both trainable).  For g = dL/dy, with W_ij = exp(-|a_i - a_j|) cos(phi_i - phi_j):
 *     dx     = W g                                                    (n x m)
 *     da_i   = - sum_jc sign(a_i - a_j) W_ij (g_ic x_jc + x_ic g_jc)   (n)
 *     dphi_i = - sum_jc exp(-|a_i - a_j|) sin(phi_i - phi_j) (g_ic x_jc + x_ic g_jc)   (n)
 * with sign(0) = 0.  Computed from scans of cos(phi) x, sin(phi) x,
 * cos(phi) g and sin(phi) g, each with the kernel's decay and summed over tied
 * anchors only.  a_sorted, perm, route: sort handle of a (route may be NULL);
 * phi: n phases, x, g: n x m (inputs, original order); dx: n x m, da, dphi: n
 * (outputs, original order, overlapping nothing).
 * ws: laplex_workspace_bytes(LAPLEX_OP_PHASED_BACKWARD, n, 0, m) bytes. */
laplex_status laplex_backward_phased(const float* a_sorted, const uint32_t* perm, const void* route, const float* phi,
                                     uint64_t n, uint32_t m, const float* x, const float* g, float* dx, float* da,
                                     float* dphi, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of the phased operator y = LAPLEX(a, phi; b, psi) x with a != b
 * (rows a, phi: n; columns b, psi: k).  For g = dL/dy, with
 * W_ij = exp(-|a_i - b_j|) cos(phi_i - psi_j):
 *     dx_j   = sum_i W_ij g_i                                         (k x m)
 *     da_i   = - sum_jc sign(a_i - b_j) W_ij g_ic x_jc,       db_j   = + sum_ic sign(a_i - b_j) W_ij g_ic x_jc
 *     dphi_i = - sum_jc exp(-|a_i - b_j|) sin(phi_i - psi_j) g_ic x_jc,
 *     dpsi_j = + sum_ic exp(-|a_i - b_j|) sin(phi_i - psi_j) g_ic x_jc
 * (sign(0) = 0), from one pass over the merge of sorted a and b.  Handles as
 * in laplex_matvec_phased; x: k x m, g: n x m (inputs, original order);
 * dx: k x m, da, dphi: n, db, dpsi: k (outputs, original order, overlapping
 * nothing).  k == 0 sets da and dphi to zero; n == 0 sets dx, db, dpsi to zero.
 * ws: laplex_workspace_bytes(LAPLEX_OP_PHASED_GENERAL_BACKWARD, n, k, m) bytes. */
laplex_status laplex_backward_phased_general(const float* a_sorted, const uint32_t* perm_a, const void* route_a,
                                             const float* phi, uint64_t n, const float* b_sorted, const uint32_t* perm_b,
                                             const void* route_b, const float* psi, uint64_t k, uint32_t m, const float* x,
                                             const float* g, float* dx, float* da, float* db, float* dphi, float* dpsi,
                                             void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of the general operator y = LAPLEX(a, b) x (rows a, n; columns b,
 * k; same section and chain rule as the symmetric backward): for g = dL/dy,
 *     dx_j = sum_i exp(-|a_i - b_j|) g_i           = LAPLEX(b, a) g   (k x m)
 *     da_i = - sum_c g_ic sum_j sign(a_i - b_j) exp(-|a_i - b_j|) x_jc   (n)
 *     db_j = - sum_c x_jc sum_i sign(b_j - a_i) exp(-|a_i - b_j|) g_ic   (k)
 * with sign(0) = 0 (an a anchor equal to a b anchor adds nothing to either
 * gradient).  All three come from one pass over the merge of sorted a and b.
 * a_sorted, perm_a, route_a: sort handle of a; b_sorted, perm_b, route_b: sort
 * handle of b (routes may be NULL); x: k x m, g: n x m (inputs, original
 * order); dx: k x m, da: n, db: k (outputs, original order, none overlapping
 * another array).  k == 0 sets da to zero; n == 0 sets dx and db to zero.
 * ws: laplex_workspace_bytes(LAPLEX_OP_GENERAL_BACKWARD, n, k, m) bytes. */
laplex_status laplex_backward_general(const float* a_sorted, const uint32_t* perm_a, const void* route_a, uint64_t n,
                                      const float* b_sorted, const uint32_t* perm_b, const void* route_b, uint64_t k,
                                      uint32_t m, const float* x, const float* g, float* dx, float* da, float* db, void* ws,
                                      size_t ws_bytes, hipStream_t stream);

/* Weighted Gram matrix M = A diag(D) A^T with A = LAPLEX(a, b) (n x k), so
 *     M_pq = sum_j D_j exp(-|a_p - b_j|) exp(-|a_q - b_j|)           (n x n),
 * computed exactly in O(n^2 + k log k) instead of O(n^2 k) (technical
 * summary, section 2.2, Gram operators): for lo <= hi the two anchors of an
 * entry, each b_j lies below lo, between them or above hi, and
 *     M = exp(-(hi - lo)) [P(lo) + C(hi) - C(lo) + Q(hi)]
 * with P(s) = sum_{b<=s} D e^{2(b-s)}, C(s) = sum_{b<=s} D (float64) and
 * Q(s) = sum_{b>s} D e^{-2(b-s)}, all taken by scans over the sorted anchors.
 * a_sorted, perm_a: sort handle of a (n); b_sorted, perm_b: sort handle of b
 * (k; for the symmetric Gram pass the handle of a again); D: k weights in the
 * original order of b.  Writes rows [row_begin, row_begin + row_count) of M,
 * rows and columns in the original order of a, row p at M + (p - row_begin) *
 * ldm (ldm >= n floats), so a matrix too large for memory can be produced in
 * slabs.  M is exactly symmetric.  k == 0 writes zeros.  Anchors must satisfy
 * |a|, |b| < 2^126 (they are doubled in float32); n <= 65535 * 1024.
 * Errors: LAPLEX_ERR_ARG for a row range past n or ldm < n.
 * ws: laplex_workspace_bytes(LAPLEX_OP_GRAM, n, k, 1) bytes. */
laplex_status laplex_gram_weighted(const float* a_sorted, const uint32_t* perm_a, uint64_t n, const float* b_sorted,
                                   const uint32_t* perm_b, uint64_t k, const float* D, uint64_t row_begin, uint64_t row_count,
                                   float* M, uint64_t ldm, void* ws, size_t ws_bytes, hipStream_t stream);

/* Short English description of a status code (static storage). */
const char* laplex_status_string(laplex_status s);

/* Opt-in launch profiler (diagnostics; not for use under stream capture).
 * laplex_profile_begin enables it for up to `capacity` kernel launches: each
 * kernel the library launches from then on is bracketed by two hipEvents
 * recorded on the stream it is launched on (events are created on the host
 * here, once).  laplex_profile_end disables it and returns the number of
 * launches recorded.  laplex_profile_get waits for record i and returns the
 * kernel's name (static storage), its duration in milliseconds and the number
 * of elements (rows) the launch processed.  The
 * profiler is process-wide state guarded by a mutex; while disabled it costs
 * one relaxed atomic load per launch. */
laplex_status laplex_profile_begin(uint32_t capacity);
uint32_t laplex_profile_end(void);
laplex_status laplex_profile_get(uint32_t i, const char** name, float* ms, uint64_t* units);

#ifdef __cplusplus
}
#endif

#endif /* LAPLEX_H */
