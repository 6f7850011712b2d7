// LAPLEX operator apply by prefix and suffix affine scans over sorted anchors
// (LAPLEX technical summary, section 2.2 "Exact Scan Algebra").
//
// Symmetric case: with anchors sorted, K = lower + upper - diagonal where
//   lower: L_i = x_i + exp(a_{i-1} - a_i) L_{i-1}      (prefix scan)
//   upper: U_i = x_i + exp(a_i - a_{i+1}) U_{i+1}      (suffix scan)
// and y[perm[i]] = exp(a_{i-1} - a_i) L_{i-1} + U_i  (strict lower + upper).
// General case a != b: the sorted a and sorted b are merged into one sequence
// (b before a on equal anchors); b elements inject x, a elements inject 0 and
// read out  y = strict forward + inclusive backward  at their position.
// Phased operator: cos(phi_i - psi_j) = cos phi_i cos psi_j + sin phi_i sin psi_j,
// so the scans carry the 2m real columns (cos psi x, sin psi x) and the
// output is recombined with cos phi_i, sin phi_i.
//
// Parallel structure (reduce-then-scan over tiles, all in fixed order so the
// result does not depend on scheduling):
//   1. per tile: gather x into sorted order and form the tile's forward and
//      backward aggregates as direct weighted sums exp(s - s_last) x and
//      exp(s_first - s) x (every weight <= 1);
//   2. one workgroup scans the tile aggregates into per-tile carries;
//   3. per tile: thread-serial recurrence over E items, wave scan by lane
//      shuffles, cross-wave combine through LDS, tile carry, and the result
//      written back to original order.
#include "laplex_kernels.hpp"
#include "laplex_scan.hpp"

namespace laplex {

// Carries for T tiles: one level when T is small, three levels otherwise.
// g_* hold the group aggregates and carries (ceil(T / 1024) x M each).
// Columns from tie_from on use the tie decay (M: no such column).
// k_tile_carry with the fewest loads per thread that cover T tiles
static hipError_t tile_carry_launch(const float* bf, const float* bb, const float2* tanch, uint64_t T, uint32_t M,
                                    uint32_t tie_from, float* cf, float* cb, hipStream_t s) {
  const uint64_t q = (T + kCarryBlock - 1) / kCarryBlock;
#define LAPLEX_CARRY(QQ) \
  LAPLEX_LAUNCH("k_tile_carry", T, s, k_tile_carry<QQ><<<M, kCarryBlock, 0, s>>>(bf, bb, tanch, T, M, tie_from, cf, cb))
  if (q <= 1)
    LAPLEX_CARRY(1);
  else if (q <= 2)
    LAPLEX_CARRY(2);
  else if (q <= 4)
    LAPLEX_CARRY(4);
  else if (q <= 8)
    LAPLEX_CARRY(8);
  else if (q <= (uint64_t)kCarryMaxQ)
    LAPLEX_CARRY(kCarryMaxQ);
  else
    return hipErrorInvalidValue;
#undef LAPLEX_CARRY
  return hipSuccess;
}

static hipError_t tile_carries(const float* bf, const float* bb, const float2* tanch, uint64_t T, uint32_t M, float* cf,
                               float* cb, float* gbf, float* gbb, float* gcf, float* gcb, float2* ganch, hipStream_t s,
                               uint32_t tie_from = ~0u) {
  // one level up to 4 tiles per thread (measured: more per thread is slower
  // than the three-level path)
  if (T <= (uint64_t)kCarryBlock * 4) {
    const hipError_t e = tile_carry_launch(bf, bb, tanch, T, M, tie_from, cf, cb, s);
    return e != hipSuccess ? e : hipGetLastError();
  }
  const uint64_t G = (T + kCarryGroup - 1) / kCarryGroup;
  if (G > kCarryMaxTiles) return hipErrorInvalidValue;  // beyond 2^24 groups of tiles
  const dim3 grid((unsigned)G, M);
  LAPLEX_LAUNCH("k_carry_up", T, s, k_carry_up<<<grid, kCarryGroup, 0, s>>>(bf, bb, tanch, T, M, tie_from, gbf, gbb, ganch));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = tile_carry_launch(gbf, gbb, ganch, G, M, tie_from, gcf, gcb, s)) != hipSuccess) return e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  LAPLEX_LAUNCH("k_carry_down", T, s,
                k_carry_down<<<grid, kCarryGroup, 0, s>>>(bf, bb, tanch, T, M, gcf, gcb, ganch, G, tie_from, cf, cb));
  return hipGetLastError();
}

// piece width for rows of m floats between x and y (16- or 8-byte vectors
// when m and both arrays allow)
static int row_piece(uint32_t m, const void* x, const void* y) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y);
  if (m % 4 == 0 && a % 16 == 0) return 4;
  if (m % 2 == 0 && a % 8 == 0) return 2;
  return 1;
}
static unsigned piece_grid(uint64_t rows, uint32_t m, int V) {
  return (unsigned)std::min<uint64_t>((rows * (m / V) + 255) / 256, 16384);
}
// xs[r] = x[perm[r]] (and phs[r] = ph[perm[r]] when ph is given), rows of m floats
static void gather_rows(const float* x, const uint32_t* perm, const float* ph, uint64_t rows, uint32_t m, float* xs, float* phs,
                        hipStream_t s) {
  const int V = row_piece(m, x, xs);
  const unsigned g = piece_grid(rows, m, V);
  const char* name = ph ? "k_gather_rows_ph" : "k_gather_rows";
  if (V == 4)
    LAPLEX_LAUNCH(name, rows, s, k_gather_rows<4><<<g, 256, 0, s>>>(x, perm, ph, rows, m, xs, phs));
  else if (V == 2)
    LAPLEX_LAUNCH(name, rows, s, k_gather_rows<2><<<g, 256, 0, s>>>(x, perm, ph, rows, m, xs, phs));
  else
    LAPLEX_LAUNCH(name, rows, s, k_gather_rows<1><<<g, 256, 0, s>>>(x, perm, ph, rows, m, xs, phs));
}
// dst[perm[r]] = src[r], rows of m floats
static void scatter_rows(const float* src, const uint32_t* perm, uint64_t rows, uint32_t m, float* dst, hipStream_t s) {
  const int V = row_piece(m, src, dst);
  const unsigned g = piece_grid(rows, m, V);
  if (V == 4)
    LAPLEX_LAUNCH("k_scatter_rows", rows, s, k_scatter_rows<4><<<g, 256, 0, s>>>(src, perm, rows, m, dst));
  else if (V == 2)
    LAPLEX_LAUNCH("k_scatter_rows", rows, s, k_scatter_rows<2><<<g, 256, 0, s>>>(src, perm, rows, m, dst));
  else
    LAPLEX_LAUNCH("k_scatter_rows", rows, s, k_scatter_rows<1><<<g, 256, 0, s>>>(src, perm, rows, m, dst));
}

// xs = x by perm (when x is given), gs = g by perm, phs = ph by perm (when
// ph is given), in one pass
static void gather_rows2(const float* x, const float* g, const uint32_t* perm, const float* ph, uint64_t rows, uint32_t m,
                         float* xs, float* gs, float* phs, hipStream_t s) {
  const int V = std::min(row_piece(m, x ? x : g, x ? xs : gs), row_piece(m, g, gs));
  const unsigned gr = piece_grid(rows, m, V);
  const char* name = !x ? (ph ? "k_gather_rows_ph" : "k_gather_rows") : (ph ? "k_gather_rows2_ph" : "k_gather_rows2");
  if (V == 4)
    LAPLEX_LAUNCH(name, rows, s, k_gather_rows2<4><<<gr, 256, 0, s>>>(x, g, perm, ph, rows, m, xs, gs, phs));
  else if (V == 2)
    LAPLEX_LAUNCH(name, rows, s, k_gather_rows2<2><<<gr, 256, 0, s>>>(x, g, perm, ph, rows, m, xs, gs, phs));
  else
    LAPLEX_LAUNCH(name, rows, s, k_gather_rows2<1><<<gr, 256, 0, s>>>(x, g, perm, ph, rows, m, xs, gs, phs));
}
// dst[perm[r]] = src[r] (rows of m floats), d1[perm[r]] = s1[r] and
// d2[perm[r]] = s2[r] (when given), in one pass
static void scatter_rows3(const float* src, const uint32_t* perm, uint64_t rows, uint32_t m, float* dst, const float* s1,
                          float* d1, const float* s2, float* d2, hipStream_t s) {
  const int V = row_piece(m, src, dst);
  const unsigned g = piece_grid(rows, m, V);
  const char* name = s2 ? "k_scatter_rows3" : s1 ? "k_scatter_rows2" : "k_scatter_rows";
  if (V == 4)
    LAPLEX_LAUNCH(name, rows, s, k_scatter_rows3<4><<<g, 256, 0, s>>>(src, perm, rows, m, dst, s1, d1, s2, d2));
  else if (V == 2)
    LAPLEX_LAUNCH(name, rows, s, k_scatter_rows3<2><<<g, 256, 0, s>>>(src, perm, rows, m, dst, s1, d1, s2, d2));
  else
    LAPLEX_LAUNCH(name, rows, s, k_scatter_rows3<1><<<g, 256, 0, s>>>(src, perm, rows, m, dst, s1, d1, s2, d2));
}

// x_sorted: w.xs already holds x in sorted order (routed, one column).
template <int C, bool PH>
static hipError_t run_sym(const ApplyWorkspace& w, const float* a_s, const uint32_t* perm, const SortRoute* route,
                          const float* phi, uint64_t n, uint32_t m, const float* x, float* y, hipStream_t s,
                          bool x_sorted = false) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int P = apply_tile(CC);
  const uint64_t T = (n + P - 1) / P;
  const uint32_t M = PH ? 2 * m : m;
  const dim3 grid((unsigned)T), block(apply_block(CC));
  const bool routed = route != nullptr && m <= kRouteMaxCols;
  const bool vec = (reinterpret_cast<uintptr_t>(a_s) & 15) == 0;
  hipError_t e;
  // x (and phi) into sorted order: along the route, or as whole rows by index
  if (routed) {
    if (!x_sorted && (e = route_forward(*route, n, m, x, w.xs, w.t0, w.t1, s)) != hipSuccess) return e;
    if (PH && (e = route_forward(*route, n, 1, phi, w.phs, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    gather_rows(x, perm, PH ? phi : nullptr, n, m, w.xs, w.phs, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  LAPLEX_LAUNCH(PH ? "k_phased_reduce" : "k_sym_reduce", n, s,
                k_sym_reduce<C, PH><<<grid, block, 0, s>>>(a_s, n, m, w.xs, w.phs, w.bf, w.bb, w.tanch, vec));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tile_carries(w.bf, w.bb, w.tanch, T, M, w.cf, w.cb, w.gbf, w.gbb, w.gcf, w.gcb, w.ganch, s)) != hipSuccess) return e;
  if (routed) {
    LAPLEX_LAUNCH(PH ? "k_phased_apply_sorted" : "k_sym_apply_sorted", n, s,
                  k_sym_apply<C, PH, false><<<grid, block, 0, s>>>(a_s, perm, w.xs, w.phs, w.cf, w.cb, w.tanch, n, m, T, w.zs, vec));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return route_inverse(*route, n, m, w.zs, y, w.t0, w.t1, s);
  }
  LAPLEX_LAUNCH(PH ? "k_phased_apply" : "k_sym_apply", n, s,
                k_sym_apply<C, PH, true><<<grid, block, 0, s>>>(a_s, perm, w.xs, w.phs, w.cf, w.cb, w.tanch, n, m, T, y, vec));
  return hipGetLastError();
}

hipError_t apply_sym_presorted(const ApplyWorkspace& w, const float* a_s, const SortRoute& route, uint64_t n, float* y,
                               hipStream_t s) {
  return run_sym<1, false>(w, a_s, nullptr, &route, nullptr, n, 1, nullptr, y, s, true);
}

// ---------------------------------------------------------------- general case: scans over b
// With few input anchors the scans can run over the sorted inputs alone
// (the split of the general sum at an output anchor that the merged scan
// makes, with the roles of the two sides exchanged): in sorted-b order
//     Fi_j = sum_{j' <= j} exp(-(b_j - b_j')) x_j'     (inclusive forward)
//     U_j  = sum_{j' >= j} exp(-(b_j' - b_j)) x_j'     (inclusive backward)
// and for an output anchor a with p = #{b_j <= a} (b before a on ties)
//     y = exp(-(a - b_{p-1})) Fi_{p-1} + exp(-(b_p - a)) U_p,
// every factor <= 1.  The output anchors need no sort: each finds p by a
// binary search, first over a sample of b staged in LDS, then inside one
// group of b.

// Fi and U of the sorted inputs (k rows of m columns), from the tile carries
// of k_sym_reduce.
template <int C>
__global__ __launch_bounds__(apply_block(C)) void k_sym_fu(const float* __restrict__ b_s, const float* __restrict__ xs,
                                                           const float* __restrict__ cfw, const float* __restrict__ cbw,
                                                           const float2* __restrict__ tanch, uint64_t k, uint32_t m, uint64_t T,
                                                           float* __restrict__ fo, float* __restrict__ uo, bool vec) {
  constexpr int E = apply_items(C);
  constexpr int NW = apply_block(C) / kWave;
  constexpr int P = apply_tile(C);
  __shared__ float s_wf[NW * C], s_wb[NW * C], s_wfs[NW], s_wbs[NW];
  const uint64_t tile = blockIdx.x;
  const uint64_t p0 = tile * P + (uint64_t)threadIdx.x * E;
  float ae[E];
  load_anchors<E>(b_s, p0, k, b_s[k - 1], vec, ae);
  const float2 ta = tanch[tile];
  const float sf = tile > 0 ? tanch[tile - 1].y : ta.x;
  const float sb = tile + 1 < T ? tanch[tile + 1].x : ta.y;
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float v[E][C], cin_f[C], cin_b[C];
    load_rows<E, C>(xs, p0, k, m, cc, true, v);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      cin_f[j] = cfw[tile * m + cc * C + j];
      cin_b[j] = cbw[tile * m + cc * C + j];
    }
    float F[E][C], U[E][C];
    tile_scan_fu<E, C, NW, false>(ae, v, cin_f, sf, cin_b, sb, s_wf, s_wfs, s_wb, s_wbs, F, U);
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < C; ++j) F[e][j] += v[e][j];
    store_rows<E, C>(fo, p0, k, m, cc, true, F);
    store_rows<E, C>(uo, p0, k, m, cc, true, U);
    __syncthreads();
  }
}

constexpr int kSearchSamples = 4096;  // b values staged in LDS per workgroup (binary search in b_s after)
constexpr int kSearchSamplesGroup = kSearchTree;  // tree slots when the search ends in a group loaded whole
constexpr int kSearchBlock = 512;
constexpr int kSearchItems = 16;      // outputs per thread, one at a time (each holds its group's S values;
                                      // more side by side measured slower: fewer waves per SIMD)
// outputs per thread of k_gen_search: more for the smallest groups, which
// leave registers for them (fewer workgroups copy the sample tree)
constexpr int search_items(int S) { return S <= 8 ? 32 : kSearchItems; }
constexpr uint32_t kSearchGroup = 8;  // b values per sample at the least (32 bytes, loaded whole)
constexpr uint32_t kSearchGroupMax = 64;

// (Fi_{q-1}, U_q) for each interval q = 0..k of the sorted inputs (zero where
// the neighbour does not exist), one column: an output in interval q reads
// both with one load.
// The same launch writes the search's sample tree (see k_gen_search) in heap
// order once, so that every search workgroup copies it contiguously instead
// of gathering one sample per group of b.
__device__ __forceinline__ uint32_t heap_node(uint32_t r, int L) {
  // sorted position r (1-based) of a complete tree of 2^L - 1 nodes: depth
  // L-1-tz(r), the (r >> (tz(r)+1))-th node of its level
  const uint32_t tz = (uint32_t)__builtin_ctz(r);
  return (1u << (L - 1 - tz)) + (r >> (tz + 1));
}
__global__ void k_gen_pairs(const float* __restrict__ fo, const float* __restrict__ uo, uint64_t k, float2* __restrict__ fu,
                            const float* __restrict__ b_s, uint64_t S, uint32_t G, float* __restrict__ tree) {
  constexpr uint32_t NS = kSearchTree;
  const uint64_t t0 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t q = t0; q <= k; q += stride) fu[q] = make_float2(q > 0 ? fo[q - 1] : 0.f, q < k ? uo[q] : 0.f);
  if (tree != nullptr)
    for (uint64_t j = t0; j + 1 < NS; j += stride)
      tree[heap_node((uint32_t)j + 1, __builtin_ctz(NS))] = j + 1 < G ? b_s[(j + 1) * S - 1] : __builtin_inff();
}

// y (n x m, original order) for the output anchors a: q = #{b_j <= a}.  The
// first G - 1 of the samples t_g = b_s[(g+1) S - 1] (the last of each group
// of S, a power of two from 8 to 64; G = ceil(k / S) <= kSearchSamplesGroup)
// sit in LDS as an implicit search tree in heap order (node 1 the root, the
// children of node i at 2i and 2i+1, in-order = sorted order, +inf past the
// samples).  Descending it counts the groups lying wholly at or below a in
// one LDS read per level; the lanes of a wave read one level's nodes, which
// are consecutive words, so the reads spread over the banks (a binary search
// over the sorted samples reads words a power of two apart, all in one bank).
// That group's S values, loaded whole, give the rest of the count and b_q;
// b_{q-1} comes from the group or, when none of it is at or below a, is the
// previous group's sample, read from its node.  One
// column takes (Fi_{q-1}, U_q) from fu, more columns the rows of fo and uo.
// Non-finite anchors raise the sort workspace's flag.
template <int S>
__global__ __launch_bounds__(kSearchBlock) void k_gen_search(const float* __restrict__ a, uint64_t n,
                                                             const float* __restrict__ b_s, uint64_t k, uint32_t G,
                                                             const float* __restrict__ fo, const float* __restrict__ uo,
                                                             const float2* __restrict__ fu, const float* __restrict__ tree, uint32_t m,
                                                             float* __restrict__ y, uint32_t* __restrict__ header) {
  static_assert(S % 4 == 0 && S <= (int)kSearchGroupMax, "groups of whole 16-byte pieces");
  constexpr uint32_t NS = kSearchSamplesGroup;
  constexpr int L = __builtin_ctz(NS);  // levels of the tree (NS - 1 nodes)
  static_assert((NS & (NS - 1)) == 0, "a complete tree");
  __shared__ float s_e[NS];  // tree nodes 1..NS-1
  auto node_of = [](uint32_t r) -> uint32_t { return heap_node(r, L); };
  const int tid = threadIdx.x;
  if (tree != nullptr) {  // the tree made once by k_gen_pairs (16-byte aligned; slot 0 unused)
    for (uint32_t j = tid; j < NS / 4; j += kSearchBlock)
      reinterpret_cast<float4*>(s_e)[j] = reinterpret_cast<const float4*>(tree)[j];
  } else {
    for (uint32_t j = tid; j + 1 < NS; j += kSearchBlock) s_e[node_of(j + 1)] = j + 1 < G ? b_s[(uint64_t)(j + 1) * S - 1] : __builtin_inff();
  }
  __syncthreads();
  constexpr int IT = search_items(S);
  const uint64_t base = (uint64_t)blockIdx.x * (kSearchBlock * IT);
  uint32_t bad = 0;
  // With small groups every output anchor of this thread is loaded up front,
  // so that no search waits on HBM for its anchor, and the outputs are
  // unrolled; larger groups take the registers that this would need.
  constexpr bool kAhead = S <= 16;
  constexpr int kUnroll = kAhead ? IT : 1;
  float a_all[kAhead ? IT : 1];
  if constexpr (kAhead) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint64_t i = base + (uint64_t)it * kSearchBlock + tid;
      a_all[it] = a[i < n ? i : n - 1];
    }
  }
#pragma unroll kUnroll
  for (int it = 0; it < IT; ++it) {
    const uint64_t i = base + (uint64_t)it * kSearchBlock + tid;
    float av;
    if constexpr (kAhead)
      av = a_all[it];
    else
      av = a[i < n ? i : n - 1];
    bad |= (i < n && bits_nonfinite(__float_as_uint(av))) ? 1u : 0u;
    uint32_t node = 1;
#pragma unroll
    for (int l = 0; l < L; ++l) node = 2 * node + (s_e[node] <= av ? 1u : 0u);
    const uint32_t cnt = node - NS;  // groups wholly at or below a: at most G - 1
    // that group's values, loaded whole (rows past k read as +inf)
    const uint64_t p = (uint64_t)cnt * S;
    float gv[S];
    if (p + S <= k) {
#pragma unroll
      for (int u = 0; u < S / 4; ++u) {
        const float4 q4 = reinterpret_cast<const float4*>(b_s + p)[u];
        gv[4 * u] = q4.x;
        gv[4 * u + 1] = q4.y;
        gv[4 * u + 2] = q4.z;
        gv[4 * u + 3] = q4.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < S; ++u) gv[u] = p + u < k ? b_s[p + u] : __builtin_inff();
    }
    uint32_t c2 = 0;
    float bl = cnt > 0 ? s_e[node_of(cnt)] : 0.f, br = 0.f;
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const bool le = gv[u] <= av;
      c2 += le ? 1u : 0u;
      bl = le ? gv[u] : bl;  // the last value <= a
    }
#pragma unroll
    for (int u = S - 1; u >= 0; --u) br = gv[u] > av ? gv[u] : br;  // the first value > a
    const uint64_t q = p + c2;  // #{b_j <= a}
    const bool left = q > 0, right = q < k;
    const float wl = left ? decay(bl - av) : 0.f;
    const float wr = right ? decay(av - br) : 0.f;
    if (i >= n) continue;
    if (m == 1) {
      const float2 f = fu[q];
      y[i] = fmaf(wr, f.y, wl * f.x);
    } else {
      const uint64_t ql = left ? q - 1 : 0, qr = right ? q : k - 1;
      for (uint32_t c = 0; c < m; ++c) {
        const float yl = left ? wl * fo[ql * m + c] : 0.f;
        y[i * m + c] = right ? fmaf(wr, uo[qr * m + c], yl) : yl;
      }
    }
  }
  if (__ballot(bad) != 0ull && lane_id() == 0) atomicOr(&header[kHdrFlags], kFlagNonFinite);
}

// The one-column search with the outputs of a workgroup taken in group
// order.  In input order every lane's group load goes to a different random
// cache line of b, so the search is bound by the rate of scattered L2
// requests.  Here each workgroup takes kLocalItems outputs per thread:
// (1) finds every output's group by the tree descent and keeps the anchor
// and group in LDS; (2) counting-sorts the outputs by group / 8 in LDS; (3)
// runs the rest of the search in that order, so neighbouring lanes load
// neighbouring groups of b and neighbouring (Fi, U) pairs, and leaves each
// result in LDS at the output's place; (4) writes y in input order.  The
// arithmetic of every output is that of k_gen_search: the same bits.
constexpr int kLocalItems = 8;                 // outputs per thread
constexpr int kLocalBins = kSearchTree / 8;    // sort bins: 8 consecutive groups each
template <int S>
__global__ __launch_bounds__(kSearchBlock) void k_gen_search_local(const float* __restrict__ a, uint64_t n,
                                                                   const float* __restrict__ b_s, uint64_t k,
                                                                   const float2* __restrict__ fu, const float* __restrict__ tree,
                                                                   float* __restrict__ y, uint32_t* __restrict__ header) {
  static_assert(S % 4 == 0 && S <= (int)kSearchGroupMax, "groups of whole 16-byte pieces");
  constexpr uint32_t NS = kSearchSamplesGroup;
  constexpr int L = __builtin_ctz(NS);
  constexpr int IT = kLocalItems;
  constexpr uint32_t CH = kSearchBlock * IT;  // outputs per workgroup
  __shared__ float s_e[NS];                     // tree nodes 1..NS-1
  __shared__ float s_a[CH];                     // anchors, then results
  __shared__ uint16_t s_g[CH];                  // group of each output
  __shared__ uint16_t s_idx[CH];                // outputs in group order
  __shared__ uint32_t s_bin[kLocalBins];
  __shared__ uint32_t s_wsum[kSearchBlock / kWave];
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  for (uint32_t j = tid; j < NS / 4; j += kSearchBlock)
    reinterpret_cast<float4*>(s_e)[j] = reinterpret_cast<const float4*>(tree)[j];
  for (uint32_t j = tid; j < (uint32_t)kLocalBins; j += kSearchBlock) s_bin[j] = 0u;
  const uint64_t base = (uint64_t)blockIdx.x * CH;
  const uint32_t count = (uint32_t)std::min<uint64_t>(CH, n - base);
  float av[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint32_t l = (uint32_t)(it * kSearchBlock + tid);
    av[it] = a[base + (l < count ? l : count - 1)];
  }
  uint32_t bad = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint32_t l = (uint32_t)(it * kSearchBlock + tid);
    bad |= (l < count && bits_nonfinite(__float_as_uint(av[it]))) ? 1u : 0u;
  }
  __syncthreads();
  // (1) groups by the tree descent; (2) bin counts
  uint32_t gl[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    uint32_t node = 1;
#pragma unroll
    for (int l = 0; l < L; ++l) node = 2 * node + (s_e[node] <= av[it] ? 1u : 0u);
    gl[it] = node - NS;
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint32_t l = (uint32_t)(it * kSearchBlock + tid);
    s_a[l] = av[it];
    s_g[l] = (uint16_t)gl[it];
    if (l < count) atomicAdd(&s_bin[gl[it] >> 3], 1u);
  }
  __syncthreads();
  // exclusive scan of the bins: two per thread, then the waves' totals
  {
    static_assert(kLocalBins == 2 * kSearchBlock, "two bins per thread");
    const uint32_t b0 = s_bin[2 * tid], b1 = s_bin[2 * tid + 1];
    const uint32_t x = wave_incl_sum_u32(b0 + b1);
    if (lane == kWave - 1) s_wsum[wid] = x;
    __syncthreads();
    uint32_t pre = 0;
    for (int w = 0; w < wid; ++w) pre += s_wsum[w];
    const uint32_t ex = pre + x - (b0 + b1);
    s_bin[2 * tid] = ex;
    s_bin[2 * tid + 1] = ex + b0;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint32_t l = (uint32_t)(it * kSearchBlock + tid);
    if (l < count) s_idx[atomicAdd(&s_bin[gl[it] >> 3], 1u)] = (uint16_t)l;
  }
  __syncthreads();
  // (3) the rest of the search in group order
  auto node_of = [](uint32_t r) -> uint32_t { return heap_node(r, L); };
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint32_t slot = (uint32_t)(it * kSearchBlock + tid);
    if (slot >= count) continue;
    const uint32_t l = s_idx[slot];
    const float v = s_a[l];
    const uint32_t cnt = s_g[l];
    const uint64_t p = (uint64_t)cnt * S;
    float gv[S];
    if (p + S <= k) {
#pragma unroll
      for (int u = 0; u < S / 4; ++u) {
        const float4 q4 = reinterpret_cast<const float4*>(b_s + p)[u];
        gv[4 * u] = q4.x;
        gv[4 * u + 1] = q4.y;
        gv[4 * u + 2] = q4.z;
        gv[4 * u + 3] = q4.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < S; ++u) gv[u] = p + u < k ? b_s[p + u] : __builtin_inff();
    }
    uint32_t c2 = 0;
    float bl = cnt > 0 ? s_e[node_of(cnt)] : 0.f, br = 0.f;
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const bool le = gv[u] <= v;
      c2 += le ? 1u : 0u;
      bl = le ? gv[u] : bl;
    }
#pragma unroll
    for (int u = S - 1; u >= 0; --u) br = gv[u] > v ? gv[u] : br;
    const uint64_t q = p + c2;
    const float wl = q > 0 ? decay(bl - v) : 0.f;
    const float wr = q < k ? decay(v - br) : 0.f;
    const float2 f = fu[q];
    s_a[l] = fmaf(wr, f.y, wl * f.x);  // each output's slot is read and written by this thread alone
  }
  __syncthreads();
  // (4) y in input order
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const uint32_t l = (uint32_t)(it * kSearchBlock + tid);
    if (l < count) y[base + l] = s_a[l];
  }
  if (__ballot(bad) != 0ull && lane_id() == 0) atomicOr(&header[kHdrFlags], kFlagNonFinite);
}

// the same search for more than kSearchSamples * kSearchGroupMax inputs: the
// group by binary search in b_s (S a power of two)
__global__ __launch_bounds__(kSearchBlock) void k_gen_search_wide(const float* __restrict__ a, uint64_t n,
                                                                  const float* __restrict__ b_s, uint64_t k, uint64_t S, uint32_t G,
                                                                  const float* __restrict__ fo, const float* __restrict__ uo,
                                                                  uint32_t m, float* __restrict__ y, uint32_t* __restrict__ header) {
  __shared__ float s_t[kSearchSamples];
  const int tid = threadIdx.x;
  for (uint32_t g = tid; g < G; g += kSearchBlock) s_t[g] = b_s[std::min<uint64_t>(k, (uint64_t)(g + 1) * S) - 1];
  __syncthreads();
  const uint64_t base = (uint64_t)blockIdx.x * (kSearchBlock * kSearchItems);
  uint32_t bad = 0;
#pragma unroll
  for (int it = 0; it < kSearchItems; ++it) {
    const uint64_t i = base + (uint64_t)it * kSearchBlock + tid;
    const float av = a[i < n ? i : n - 1];
    bad |= (i < n && bits_nonfinite(__float_as_uint(av))) ? 1u : 0u;
    uint32_t cnt = 0;
    for (uint32_t step = kSearchSamples; step >= 1; step >>= 1) {
      const uint32_t t = cnt + step;
      cnt = (t <= G && s_t[(t < G ? t : G) - 1] <= av) ? t : cnt;
    }
    const uint64_t p = std::min<uint64_t>(k, (uint64_t)cnt * S);
    uint64_t c2 = 0;
    for (uint64_t step = S; step >= 1; step >>= 1) {
      const uint64_t t = p + c2 + step;
      c2 = (t <= k && c2 + step <= S && b_s[(t < k ? t : k) - 1] <= av) ? c2 + step : c2;
    }
    const uint64_t q = p + c2;
    const bool left = q > 0, right = q < k;
    const uint64_t ql = left ? q - 1 : 0, qr = right ? q : k - 1;
    const float wl = left ? decay(b_s[ql] - av) : 0.f;
    const float wr = right ? decay(av - b_s[qr]) : 0.f;
    if (i >= n) continue;
    for (uint32_t c = 0; c < m; ++c) {
      const float yl = left ? wl * fo[ql * m + c] : 0.f;
      y[i * m + c] = right ? fmaf(wr, uo[qr * m + c], yl) : yl;
    }
  }
  if (__ballot(bad) != 0ull && lane_id() == 0) atomicOr(&header[kHdrFlags], kFlagNonFinite);
}

template <int C>
static hipError_t run_general_search(const ApplyWorkspace& w, float* fo, float* uo, float2* fu, const float* a, uint64_t n, const float* b_s,
                                     const uint32_t* perm_b, uint64_t k, uint32_t m, const float* x, float* y, uint32_t* header,
                                     hipStream_t s) {
  constexpr int P = apply_tile(C);
  const uint64_t T = (k + P - 1) / P;
  const bool vec = (reinterpret_cast<uintptr_t>(b_s) & 15) == 0;
  hipError_t e;
  gather_rows(x, perm_b, nullptr, k, m, w.xs, nullptr, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  LAPLEX_LAUNCH("k_sym_reduce", k, s,
                k_sym_reduce<C, false><<<dim3((unsigned)T), dim3(apply_block(C)), 0, s>>>(b_s, k, m, w.xs, nullptr, w.bf, w.bb,
                                                                                         w.tanch, vec));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tile_carries(w.bf, w.bb, w.tanch, T, m, w.cf, w.cb, w.gbf, w.gbb, w.gcf, w.gcb, w.ganch, s)) != hipSuccess) return e;
  LAPLEX_LAUNCH("k_sym_fu", k, s,
                k_sym_fu<C><<<dim3((unsigned)T), dim3(apply_block(C)), 0, s>>>(b_s, w.xs, w.cf, w.cb, w.tanch, k, m, T, fo, uo, vec));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  uint64_t S = kSearchGroup;
  while ((k + S - 1) / S > (uint64_t)kSearchSamplesGroup) S <<= 1;
  if (S > kSearchGroupMax)
    while ((k + S - 1) / S > (uint64_t)kSearchSamples) S <<= 1;
  const uint32_t G = (uint32_t)((k + S - 1) / S);
  const uint64_t per_block = (uint64_t)kSearchBlock * (S <= kSearchGroupMax ? search_items((int)S) : kSearchItems);
  const unsigned blocks = (unsigned)((n + per_block - 1) / per_block);
  // one column: the pairs and the sample tree, after the pairs in fu's table
  float* tree = m == 1 && S <= kSearchGroupMax ? search_tree(fu, k) : nullptr;
  if (m == 1 && S <= kSearchGroupMax) {
    LAPLEX_LAUNCH("k_gen_pairs", k + 1, s,
                  k_gen_pairs<<<(unsigned)std::min<uint64_t>((std::max<uint64_t>(k + 1, kSearchTree) + 255) / 256, 4096), 256, 0, s>>>(
                      fo, uo, k, fu, b_s, S, G, tree));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const unsigned lblocks = (unsigned)((n + (uint64_t)kSearchBlock * kLocalItems - 1) / ((uint64_t)kSearchBlock * kLocalItems));
#define LAPLEX_SEARCH(SS)                                                                                             \
  if (m == 1)                                                                                                         \
    LAPLEX_LAUNCH("k_gen_search", n, s,                                                                               \
                  k_gen_search_local<SS><<<lblocks, kSearchBlock, 0, s>>>(a, n, b_s, k, fu, tree, y, header));         \
  else                                                                                                                \
    LAPLEX_LAUNCH("k_gen_search", n, s, k_gen_search<SS><<<blocks, kSearchBlock, 0, s>>>(a, n, b_s, k, G, fo, uo, fu, tree, m, y, header))
  if (S == 8)
    LAPLEX_SEARCH(8);
  else if (S == 16)
    LAPLEX_SEARCH(16);
  else if (S == 32)
    LAPLEX_SEARCH(32);
  else if (S == 64)
    LAPLEX_SEARCH(64);
  else
    LAPLEX_LAUNCH("k_gen_search", n, s,
                  k_gen_search_wide<<<blocks, kSearchBlock, 0, s>>>(a, n, b_s, k, S, G, fo, uo, m, y, header));
#undef LAPLEX_SEARCH
  return hipGetLastError();
}

hipError_t apply_general_search(const ApplyWorkspace& w, float* fo, float* uo, float2* fu, const float* a, uint64_t n, const float* b_s,
                                const uint32_t* perm_b, uint64_t k, uint32_t m, const float* x, float* y, uint32_t* header,
                                hipStream_t s) {
  switch (column_chunk(m)) {
    case 8: return run_general_search<8>(w, fo, uo, fu, a, n, b_s, perm_b, k, m, x, y, header, s);
    case 4: return run_general_search<4>(w, fo, uo, fu, a, n, b_s, perm_b, k, m, x, y, header, s);
    case 2: return run_general_search<2>(w, fo, uo, fu, a, n, b_s, perm_b, k, m, x, y, header, s);
    default: return run_general_search<1>(w, fo, uo, fu, a, n, b_s, perm_b, k, m, x, y, header, s);
  }
}

hipError_t apply_sym(const ApplyWorkspace& w, Variant var, const float* a_s, const uint32_t* perm, const SortRoute* route,
                     const float* phi, uint64_t n, uint32_t m, const float* x, float* y, hipStream_t s) {
  const bool ph = var == Variant::Phased;
#define LAPLEX_SYM(CW)                                                               \
  return ph ? run_sym<CW, true>(w, a_s, perm, route, phi, n, m, x, y, s)          \
            : run_sym<CW, false>(w, a_s, perm, route, phi, n, m, x, y, s)
  switch (ph ? phased_chunk(m) : column_chunk(m)) {
    case 8: LAPLEX_SYM(8);
    case 4: LAPLEX_SYM(4);
    case 2: LAPLEX_SYM(2);
    default: LAPLEX_SYM(1);
  }
#undef LAPLEX_SYM
}

// This thread's E consecutive elements of a merged tile (s_a: the tile's na a
// anchors, s_b: its nb b anchors, b first on equal anchors; sp0: global index
// of the tile's first a and first b): anchor (pad past the end), kind (0 pad,
// 1 a, 2 b), global index into a_s or b_s, and the number of b elements that
// precede the element in the whole merge.  Written without branches: every
// per-element value is selected from the same predicate.
template <int E>
__device__ __forceinline__ void merge_tile_items(const float* s_a, const float* s_b, uint32_t na, uint32_t nb, uint2 sp0,
                                                 float pad, float (&ae)[E], int (&kind)[E], uint32_t (&idx)[E],
                                                 uint32_t (&bbefore)[E]) {
  const uint32_t tot = na + nb;
  const uint32_t dd = std::min<uint32_t>(tot, (uint32_t)threadIdx.x * E);
  uint32_t lo = dd > nb ? dd - nb : 0u, hi = std::min(dd, na);
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (s_a[mid] < s_b[dd - 1 - mid])
      lo = mid + 1;
    else
      hi = mid;
  }
  uint32_t ii = lo, jj = dd - lo;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool real = (uint32_t)threadIdx.x * E + e < tot;
    const float va = ii < na ? s_a[ii] : INFINITY;
    const float vb = jj < nb ? s_b[jj] : INFINITY;
    const bool take_b = real && (jj < nb) && (vb <= va);
    const bool take_a = real && !take_b;
    ae[e] = take_b ? vb : (take_a ? va : pad);
    kind[e] = take_b ? 2 : (take_a ? 1 : 0);
    idx[e] = take_b ? sp0.y + jj : (take_a ? sp0.x + ii : 0u);
    bbefore[e] = sp0.y + jj;
    jj += take_b ? 1u : 0u;
    ii += take_a ? 1u : 0u;
  }
}

// ---------------------------------------------------------------- backward (symmetric)
// With y = K x and an upstream gradient g = dL/dy (technical summary,
// section 2.3: the operator is differentiable in its anchors), the chain rule
// on K_ij = exp(-|a_i - a_j|) gives
//     dx   = K g,
//     da_i = - sum_c [ g_ic S(x_c)_i + x_ic S(g_c)_i ],
//     S(v)_i = sum_j sign(a_i - a_j) exp(-|a_i - a_j|) v_j   (sign(0) = 0).
// In sorted order S(v) = (F - F0) - (U - U0): F, U are the strict forward and
// inclusive backward scans of v (tied anchors counted with weight 1), F0, U0
// the same scans with the tie decay (sums over tied anchors only), so the
// differences keep exactly the anchors strictly below and above.
//
// Summary columns (M = 4m): [0, m) x and [m, 2m) g with the kernel's decay,
// [2m, 3m) x and [3m, 4m) g with the tie decay.
template <int C>
__device__ __forceinline__ uint32_t bwdcol(uint32_t m, uint32_t cc, int j) {
  const uint32_t mode = (uint32_t)j / (2 * C), which = ((uint32_t)j / C) % 2, col = (uint32_t)j % C;
  return mode * 2 * m + which * m + cc * C + col;
}

// Gathered inputs (or their rows moved by route) -> tile aggregates of x and g
// under both decays, as direct weighted sums.  PAIR (one column): x and g
// arrive interleaved as rows (x_i, g_i) in xs.
template <int C, bool PAIR>
__global__ __launch_bounds__(bwd_block(C)) void k_bwd_reduce(const float* __restrict__ a_s, const float* __restrict__ xs,
                                                                   const float* __restrict__ gs, uint64_t n, uint32_t m,
                                                                   float* __restrict__ bf, float* __restrict__ bb,
                                                                   float2* __restrict__ tanch, bool vec) {
  constexpr int CC = 4 * C;
  constexpr int E = bwd_items(C);
  constexpr int BLOCK = bwd_block(C);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_red[2 * NW * CC];
  const uint32_t M = 4 * m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t lo = tile * P;
  const uint64_t hi = std::min<uint64_t>(n, lo + P);
  const float s_first = a_s[lo], s_last = a_s[hi - 1];
  if (tid == 0) tanch[tile] = make_float2(s_first, s_last);
  const uint64_t p0 = lo + (uint64_t)tid * E;
  float ae[E], wf[E], wb[E], tf[E], tb[E];
  load_anchors<E>(a_s, p0, n, s_last, vec, ae);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool valid = p0 + e < n;
    wf[e] = valid ? decay(ae[e] - s_last) : 0.f;
    wb[e] = valid ? decay(s_first - ae[e]) : 0.f;
    tf[e] = valid ? decay_m<true>(ae[e] - s_last) : 0.f;
    tb[e] = valid ? decay_m<true>(s_first - ae[e]) : 0.f;
  }
  static_assert(!PAIR || C == 1, "pairs carry one column");
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float xv[E][C], gv[E][C];
    if constexpr (PAIR) {
      float xg[E][2];
      load_rows<E, 2>(xs, p0, n, 2, 0, true, xg);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        xv[e][0] = xg[e][0];
        gv[e][0] = xg[e][1];
      }
    } else {
      load_rows<E, C>(xs, p0, n, m, cc, true, xv);
      load_rows<E, C>(gs, p0, n, m, cc, true, gv);
    }
    float sf[CC], sb[CC];
#pragma unroll
    for (int j = 0; j < CC; ++j) sf[j] = sb[j] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        sf[j] = fmaf(wf[e], xv[e][j], sf[j]);
        sf[C + j] = fmaf(wf[e], gv[e][j], sf[C + j]);
        sf[2 * C + j] = fmaf(tf[e], xv[e][j], sf[2 * C + j]);
        sf[3 * C + j] = fmaf(tf[e], gv[e][j], sf[3 * C + j]);
        sb[j] = fmaf(wb[e], xv[e][j], sb[j]);
        sb[C + j] = fmaf(wb[e], gv[e][j], sb[C + j]);
        sb[2 * C + j] = fmaf(tb[e], xv[e][j], sb[2 * C + j]);
        sb[3 * C + j] = fmaf(tb[e], gv[e][j], sb[3 * C + j]);
      }
    }
    int writer = 0;
    block_sum2<CC, NW>(sf, sb, s_red, writer);
    if (writer) {
      float f = 0.f, b = 0.f;
      for (int w = 0; w < NW; ++w) {
        f += s_red[(0 * NW + w) * CC + tid];
        b += s_red[(1 * NW + w) * CC + tid];
      }
      const uint32_t col = bwdcol<C>(m, cc, tid);
      bf[tile * M + col] = f;
      bb[tile * M + col] = b;
    }
    __syncthreads();
  }
}

// Tile scans of (x, g) under both decays -> dx = K g (rows in sorted order)
// and da (sorted order).  By linearity da_i = -(A_i - A0_i) with
// A = sum_c g_c (F - U)(x_c) + x_c (F - U)(g_c) under the kernel's decay and A0
// the same under the tie decay.  One column scans both decays in one pass
// (four columns, the tie half first); wider chunks run the tie scan first and
// keep only its per-element sum through the second.  PAIR (one column): x and g arrive
// interleaved as rows (x_i, g_i) in xs.
template <int C, bool PAIR>
__global__ __launch_bounds__(bwd_block(C)) void k_bwd_apply(const float* __restrict__ a_s, const float* __restrict__ xs, const float* __restrict__ gs,
                 const float* __restrict__ cfw, const float* __restrict__ cbw, const float2* __restrict__ tanch,
                 uint64_t n, uint32_t m, uint64_t T, float* __restrict__ dxs, float* __restrict__ das, bool vec) {
  constexpr int CC = 2 * C;  // columns of one scan (x then g)
  constexpr int E = bwd_items(C);
  constexpr int BLOCK = bwd_block(C);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_wf[NW * 2 * CC], s_wb[NW * 2 * CC], s_wfs[NW], s_wbs[NW];
  const uint32_t M = 4 * m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t p0 = tile * P + (uint64_t)tid * E;
  float ae[E];
  load_anchors<E>(a_s, p0, n, a_s[n - 1], vec, ae);
  const float2 ta = tanch[tile];
  const float sf = tile > 0 ? tanch[tile - 1].y : ta.x;
  const float sb = tile + 1 < T ? tanch[tile + 1].x : ta.y;
  static_assert(!PAIR || C == 1, "pairs carry one column");
  float acc[E], acc0[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = acc0[e] = 0.f;
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float v[E][CC];
    {
      float xv[E][C], gv[E][C];
      if constexpr (PAIR) {
        float xg[E][2];
        load_rows<E, 2>(xs, p0, n, 2, 0, true, xg);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          xv[e][0] = xg[e][0];
          gv[e][0] = xg[e][1];
        }
      } else {
        load_rows<E, C>(xs, p0, n, m, cc, true, xv);
        load_rows<E, C>(gs, p0, n, m, cc, true, gv);
      }
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          v[e][j] = xv[e][j];
          v[e][C + j] = gv[e][j];
        }
    }
    if constexpr (C > 1) {
      // wider chunks: the tie scan, then the kernel's scan (one mixed scan of
      // twice the columns would hold too many registers)
      float ct_f[CC], ct_b[CC];
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        ct_f[j] = cfw[tile * M + bwdcol<C>(m, cc, CC + j)];
        ct_b[j] = cbw[tile * M + bwdcol<C>(m, cc, CC + j)];
      }
      float F0[E][CC], U0[E][CC];
      tile_scan_fu<E, CC, NW, true>(ae, v, ct_f, sf, ct_b, sb, s_wf, s_wfs, s_wb, s_wbs, F0, U0);
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          acc0[e] = fmaf(v[e][C + j], F0[e][j] - U0[e][j], acc0[e]);
          acc0[e] = fmaf(v[e][j], F0[e][C + j] - U0[e][C + j], acc0[e]);
        }
      __syncthreads();  // the second scan reuses the wave summaries
      float ce_f[CC], ce_b[CC];
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        ce_f[j] = cfw[tile * M + bwdcol<C>(m, cc, j)];
        ce_b[j] = cbw[tile * M + bwdcol<C>(m, cc, j)];
      }
      float F[E][CC], U[E][CC];
      tile_scan_fu<E, CC, NW, false>(ae, v, ce_f, sf, ce_b, sb, s_wf, s_wfs, s_wb, s_wbs, F, U);
      float dx[E][C];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          acc[e] = fmaf(v[e][C + j], F[e][j] - U[e][j], acc[e]);
          acc[e] = fmaf(v[e][j], F[e][C + j] - U[e][C + j], acc[e]);
          dx[e][j] = F[e][C + j] + U[e][C + j];
        }
      store_rows<E, C>(dxs, p0, n, m, cc, true, dx);
    } else {
      // one column: one scan of [x, g | x, g], the first half with the tie
      // decay (sums over tied anchors, F0 and U0), the second with the
      // kernel's decay
      float v2[E][2 * CC], c2f[2 * CC], c2b[2 * CC];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < CC; ++j) v2[e][j] = v2[e][CC + j] = v[e][j];
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        c2f[j] = cfw[tile * M + bwdcol<C>(m, cc, CC + j)];
        c2b[j] = cbw[tile * M + bwdcol<C>(m, cc, CC + j)];
        c2f[CC + j] = cfw[tile * M + bwdcol<C>(m, cc, j)];
        c2b[CC + j] = cbw[tile * M + bwdcol<C>(m, cc, j)];
      }
      float F2[E][2 * CC], U2[E][2 * CC];
      tile_scan_fu_mix<E, 2 * CC, NW, CC>(ae, v2, c2f, sf, c2b, sb, s_wf, s_wfs, s_wb, s_wbs, F2, U2);
      float dx[E][C];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          acc0[e] = fmaf(v[e][C + j], F2[e][j] - U2[e][j], acc0[e]);
          acc0[e] = fmaf(v[e][j], F2[e][C + j] - U2[e][C + j], acc0[e]);
          acc[e] = fmaf(v[e][C + j], F2[e][CC + j] - U2[e][CC + j], acc[e]);
          acc[e] = fmaf(v[e][j], F2[e][CC + C + j] - U2[e][CC + C + j], acc[e]);
          dx[e][j] = F2[e][CC + C + j] + U2[e][CC + C + j];
        }
      store_rows<E, C>(dxs, p0, n, m, cc, true, dx);
    }
    __syncthreads();
  }
  float dav[E][1];
#pragma unroll
  for (int e = 0; e < E; ++e) dav[e][0] = acc0[e] - acc[e];
  store_rows<E, 1>(das, p0, n, 1, 0, true, dav);
}

// dst[perm[r]] = src[r] for rows of m floats (rows in sorted order -> original)
static unsigned rows_grid(uint64_t rows) { return (unsigned)std::min<uint64_t>((rows + 255) / 256, 8192); }

template <int C>
// xs_sorted: x already in sorted order (kept by a one-call forward); then
// only g is moved into sorted order.
static hipError_t run_bwd_sym(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm, const SortRoute* route,
                              uint64_t n, uint32_t m, const float* x, const float* g, float* dx, float* da, hipStream_t s,
                              const float* xs_sorted = nullptr) {
  const ApplyWorkspace& w = bw.w;
  const float* xs = xs_sorted ? xs_sorted : w.xs;
  constexpr int P = bwd_tile(C);
  const uint64_t T = (n + P - 1) / P;
  const uint32_t M = 4 * m;
  const dim3 grid((unsigned)T), block(bwd_block(C));
  const bool routed = route != nullptr && m <= kRouteMaxCols;
  const bool vec = (reinterpret_cast<uintptr_t>(a_s) & 15) == 0;
  hipError_t e;
  if (C == 1 && m == 1 && routed && !xs_sorted) {
    // one column: x and g travel as pairs (one read of each route table for
    // both); dx and da go back one by one (an inverse pass of pairs stages
    // twice the LDS and fits half the workgroups)
    if ((e = route_forward_pair(*route, n, x, g, w.xs, w.t0, w.t1, s)) != hipSuccess) return e;
    LAPLEX_LAUNCH("k_bwd_reduce", n, s,
                  k_bwd_reduce<C, C == 1><<<grid, block, 0, s>>>(a_s, w.xs, nullptr, n, m, w.bf, w.bb, w.tanch, vec));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = tile_carries(w.bf, w.bb, w.tanch, T, M, w.cf, w.cb, w.gbf, w.gbb, w.gcf, w.gcb, w.ganch, s, 2 * m)) !=
        hipSuccess)
      return e;
    LAPLEX_LAUNCH("k_bwd_apply", n, s,
                  k_bwd_apply<C, C == 1><<<grid, block, 0, s>>>(a_s, w.xs, nullptr, w.cf, w.cb, w.tanch, n, m, T, w.zs, bw.das,
                                                                vec));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = route_inverse(*route, n, 1, w.zs, dx, w.t0, w.t1, s)) != hipSuccess) return e;
    return route_inverse(*route, n, 1, bw.das, da, w.t0, w.t1, s);
  }
  if (routed) {
    if (!xs_sorted && (e = route_forward(*route, n, m, x, w.xs, w.t0, w.t1, s)) != hipSuccess) return e;
    if ((e = route_forward(*route, n, m, g, bw.gs, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    gather_rows2(xs_sorted ? nullptr : x, g, perm, nullptr, n, m, w.xs, bw.gs, nullptr, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  LAPLEX_LAUNCH("k_bwd_reduce", n, s,
                k_bwd_reduce<C, false><<<grid, block, 0, s>>>(a_s, xs, bw.gs, n, m, w.bf, w.bb, w.tanch, vec));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tile_carries(w.bf, w.bb, w.tanch, T, M, w.cf, w.cb, w.gbf, w.gbb, w.gcf, w.gcb, w.ganch, s, 2 * m)) != hipSuccess)
    return e;
  LAPLEX_LAUNCH("k_bwd_apply", n, s,
                k_bwd_apply<C, false><<<grid, block, 0, s>>>(a_s, xs, bw.gs, w.cf, w.cb, w.tanch, n, m, T, w.zs, bw.das, vec));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (routed) {
    if ((e = route_inverse(*route, n, m, w.zs, dx, w.t0, w.t1, s)) != hipSuccess) return e;
    return route_inverse(*route, n, 1, bw.das, da, w.t0, w.t1, s);
  }
  scatter_rows3(w.zs, perm, n, m, dx, bw.das, da, nullptr, nullptr, s);
  return hipGetLastError();
}

hipError_t backward_sym(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm, const SortRoute* route,
                        uint64_t n, uint32_t m, const float* x, const float* g, float* dx, float* da, hipStream_t s,
                        const float* xs_sorted) {
  switch (column_chunk(m)) {
    case 8: return run_bwd_sym<8>(bw, a_s, perm, route, n, m, x, g, dx, da, s, xs_sorted);
    case 4: return run_bwd_sym<4>(bw, a_s, perm, route, n, m, x, g, dx, da, s, xs_sorted);
    case 2: return run_bwd_sym<2>(bw, a_s, perm, route, n, m, x, g, dx, da, s, xs_sorted);
    default: return run_bwd_sym<1>(bw, a_s, perm, route, n, m, x, g, dx, da, s, xs_sorted);
  }
}

// ---------------------------------------------------------------- phased backward
// Backward of the symmetric phased operator y_i = sum_j K_ij cos(phi_i - phi_j) x_j
// (K_ij = exp(-|a_i - a_j|)) for g = dL/dy.  Per input column four real columns
// are scanned: cx = cos(phi) x, sx = sin(phi) x, cg = cos(phi) g, sg = sin(phi) g.
// With K(v) = F + U and S(v) = (F - U) - (F0 - U0) as in the symmetric backward
// (angle-difference identity applied to every entry and its derivatives):
//     dx_i   = cos phi_i K(cg)_i + sin phi_i K(sg)_i,
//     da_i   = -sum_c [ g (cos S(cx) + sin S(sx)) + x (cos S(cg) + sin S(sg)) ]_i,
//     dphi_i =  sum_c [ -g (sin K(cx) - cos K(sx)) + x (cos K(sg) - sin K(cg)) ]_i.
// Summary columns (M = 8m): kind q (cx, sx, cg, sg) at [q m, (q + 1) m) with
// the kernel's decay, and 4m + the same with the tie decay.
template <int C>
__device__ __forceinline__ uint32_t pbwdcol(uint32_t m, uint32_t cc, int j) {
  const uint32_t mode = (uint32_t)j / (4 * C), kind = ((uint32_t)j / C) % 4, col = (uint32_t)j % C;
  return mode * 4 * m + kind * m + cc * C + col;
}
constexpr int pbwd_items(int c) { return apply_items(4 * c); }
constexpr int pbwd_block(int c) { return apply_block(4 * c); }

// Column slices of a tile's rows staged in LDS.  The phased backward scans
// one input column per pass; reading that column straight from the
// row-major arrays would fetch every row once per column.  Instead the
// tile's rows [lo, lo + P), columns [c0, c0 + w) (w <= kStageCols) are
// loaded once, as 16-byte pieces when the layout allows, and kept column by
// column: s[j * P + r] = x[(lo + r) * m + c0 + j], zero past row n; a
// thread's E consecutive rows of one column are then one LDS vector read.
constexpr uint32_t kStageCols = 4;
template <int P, int BLOCK>
__device__ __forceinline__ void stage_cols(const float* __restrict__ x, uint64_t lo, uint64_t n, uint32_t m, uint32_t c0,
                                           uint32_t w, bool vec4, float* __restrict__ s) {
  const uint32_t rows = (uint32_t)std::min<uint64_t>((uint64_t)P, n - lo);
  if (vec4 && w == 4) {
    for (uint32_t r = threadIdx.x; r < (uint32_t)P; r += BLOCK) {
      const float4 q = r < rows ? *reinterpret_cast<const float4*>(x + (lo + r) * m + c0) : make_float4(0.f, 0.f, 0.f, 0.f);
      s[0 * P + r] = q.x;
      s[1 * P + r] = q.y;
      s[2 * P + r] = q.z;
      s[3 * P + r] = q.w;
    }
  } else {
    for (uint32_t q = threadIdx.x; q < (uint32_t)P * w; q += BLOCK) {
      const uint32_t r = q / w, j = q - r * w;
      s[j * P + r] = r < rows ? x[(lo + r) * m + c0 + j] : 0.f;
    }
  }
}
// The reverse: rows [lo, lo + P) (up to n), columns [c0, c0 + w) of y from s.
template <int P, int BLOCK>
__device__ __forceinline__ void unstage_cols(float* __restrict__ y, uint64_t lo, uint64_t n, uint32_t m, uint32_t c0, uint32_t w,
                                             bool vec4, const float* __restrict__ s) {
  const uint32_t rows = (uint32_t)std::min<uint64_t>((uint64_t)P, n - lo);
  if (vec4 && w == 4) {
    for (uint32_t r = threadIdx.x; r < rows; r += BLOCK)
      *reinterpret_cast<float4*>(y + (lo + r) * m + c0) = make_float4(s[r], s[P + r], s[2 * P + r], s[3 * P + r]);
  } else {
    for (uint32_t q = threadIdx.x; q < rows * w; q += BLOCK) {
      const uint32_t r = q / w, j = q - r * w;
      y[(lo + r) * m + c0 + j] = s[j * P + r];
    }
  }
}
// a thread's E consecutive rows (local p) of staged column j
template <int E, int P>
__device__ __forceinline__ void staged_rows(const float* s, uint32_t j, uint32_t p, float (&v)[E][1]) {
  if constexpr (E == 4) {
    const float4 q = *reinterpret_cast<const float4*>(s + j * P + p);
    v[0][0] = q.x;
    v[1][0] = q.y;
    v[2][0] = q.z;
    v[3][0] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e][0] = s[j * P + p + e];
  }
}

// the four scanned values of element e, column j
template <int E, int C>
__device__ __forceinline__ void phased_quad(const float (&cs)[E], const float (&sn)[E], const float (&xv)[E][C],
                                            const float (&gv)[E][C], float (&v)[E][4 * C]) {
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int j = 0; j < C; ++j) {
      v[e][j] = cs[e] * xv[e][j];
      v[e][C + j] = sn[e] * xv[e][j];
      v[e][2 * C + j] = cs[e] * gv[e][j];
      v[e][3 * C + j] = sn[e] * gv[e][j];
    }
}

template <int C>
__global__ __launch_bounds__(pbwd_block(C)) void k_pbwd_reduce(const float* __restrict__ a_s, const float* __restrict__ xs,
                                                               const float* __restrict__ gs, const float* __restrict__ phs,
                                                               uint64_t n, uint32_t m, float* __restrict__ bf,
                                                               float* __restrict__ bb, float2* __restrict__ tanch, bool vec) {
  constexpr int CC = 8 * C;
  constexpr int E = pbwd_items(C);
  constexpr int BLOCK = pbwd_block(C);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_red[2 * NW * CC];
  const uint32_t M = 8 * m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t lo = tile * P;
  const uint64_t hi = std::min<uint64_t>(n, lo + P);
  const float s_first = a_s[lo], s_last = a_s[hi - 1];
  if (tid == 0) tanch[tile] = make_float2(s_first, s_last);
  const uint64_t p0 = lo + (uint64_t)tid * E;
  float ae[E], ph[E], cs[E], sn[E], wf[E], wb[E], tf[E], tb[E];
  load_anchors<E>(a_s, p0, n, s_last, vec, ae);
  load_anchors<E>(phs, p0, n, 0.f, true, ph);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    sincosf(ph[e], &sn[e], &cs[e]);
    const bool valid = p0 + e < n;
    wf[e] = valid ? decay(ae[e] - s_last) : 0.f;
    wb[e] = valid ? decay(s_first - ae[e]) : 0.f;
    tf[e] = valid ? decay_m<true>(ae[e] - s_last) : 0.f;
    tb[e] = valid ? decay_m<true>(s_first - ae[e]) : 0.f;
  }
  static_assert(C == 1, "one input column per pass");
  __shared__ float s_x[kStageCols * P], s_g[kStageCols * P];
  const bool vec4 = (m % 4 == 0) && (reinterpret_cast<uintptr_t>(xs) % 16 == 0) && (reinterpret_cast<uintptr_t>(gs) % 16 == 0);
  // With 16-byte row pieces the next slice's pieces are loaded into
  // registers while the current slice is reduced, and written to LDS after
  // the barrier that ends the current slice's reads.
  static_assert(kStageCols == 4 && P % BLOCK == 0, "one 16-byte piece per row and slice");
  constexpr int SR = P / BLOCK;  // rows of a slice per thread
  const uint32_t rows = (uint32_t)std::min<uint64_t>((uint64_t)P, n - lo);
  float4 nx[SR], ng[SR];
  auto fetch = [&](uint32_t c0) {
#pragma unroll
    for (int r = 0; r < SR; ++r) {
      const uint32_t row = (uint32_t)(r * BLOCK + tid);
      const bool ok = row < rows;
      nx[r] = ok ? *reinterpret_cast<const float4*>(xs + (lo + row) * m + c0) : make_float4(0.f, 0.f, 0.f, 0.f);
      ng[r] = ok ? *reinterpret_cast<const float4*>(gs + (lo + row) * m + c0) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if (vec4) fetch(0);
  for (uint32_t cc = 0; cc < m; ++cc) {
    const uint32_t j0 = cc % kStageCols;
    if (j0 == 0) {  // the next slice of columns, loaded once for the whole tile
      __syncthreads();
      if (vec4) {
#pragma unroll
        for (int r = 0; r < SR; ++r) {
          const uint32_t row = (uint32_t)(r * BLOCK + tid);
          s_x[0 * P + row] = nx[r].x;
          s_x[1 * P + row] = nx[r].y;
          s_x[2 * P + row] = nx[r].z;
          s_x[3 * P + row] = nx[r].w;
          s_g[0 * P + row] = ng[r].x;
          s_g[1 * P + row] = ng[r].y;
          s_g[2 * P + row] = ng[r].z;
          s_g[3 * P + row] = ng[r].w;
        }
        if (cc + kStageCols < m) fetch(cc + kStageCols);
      } else {
        const uint32_t w = std::min<uint32_t>(kStageCols, m - cc);
        stage_cols<P, BLOCK>(xs, lo, n, m, cc, w, false, s_x);
        stage_cols<P, BLOCK>(gs, lo, n, m, cc, w, false, s_g);
      }
      __syncthreads();
    }
    float xv[E][C], gv[E][C], v[E][4 * C];
    staged_rows<E, P>(s_x, j0, (uint32_t)tid * E, xv);
    staged_rows<E, P>(s_g, j0, (uint32_t)tid * E, gv);
    phased_quad<E, C>(cs, sn, xv, gv, v);
    float sf[CC], sb[CC];
#pragma unroll
    for (int j = 0; j < CC; ++j) sf[j] = sb[j] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < 4 * C; ++j) {
        sf[j] = fmaf(wf[e], v[e][j], sf[j]);
        sb[j] = fmaf(wb[e], v[e][j], sb[j]);
        sf[4 * C + j] = fmaf(tf[e], v[e][j], sf[4 * C + j]);
        sb[4 * C + j] = fmaf(tb[e], v[e][j], sb[4 * C + j]);
      }
    int writer = 0;
    block_sum2<CC, NW>(sf, sb, s_red, writer);
    if (writer) {
      float f = 0.f, b = 0.f;
      for (int w = 0; w < NW; ++w) {
        f += s_red[(0 * NW + w) * CC + tid];
        b += s_red[(1 * NW + w) * CC + tid];
      }
      const uint32_t col = pbwdcol<C>(m, cc, tid);
      bf[tile * M + col] = f;
      bb[tile * M + col] = b;
    }
    __syncthreads();
  }
}

template <int C>
__global__ __launch_bounds__(pbwd_block(C)) void k_pbwd_apply(const float* __restrict__ a_s, const float* __restrict__ xs,
                                                              const float* __restrict__ gs, const float* __restrict__ phs,
                                                              const float* __restrict__ cfw, const float* __restrict__ cbw,
                                                              const float2* __restrict__ tanch, uint64_t n, uint32_t m, uint64_t T,
                                                              float* __restrict__ dxs, float* __restrict__ das,
                                                              float* __restrict__ dphs, bool vec) {
  constexpr int CC = 4 * C;  // columns of one scan (cx, sx, cg, sg)
  constexpr int E = pbwd_items(C);
  constexpr int BLOCK = pbwd_block(C);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_wf[NW * 2 * CC], s_wb[NW * 2 * CC], s_wfs[NW], s_wbs[NW];
  const uint32_t M = 8 * m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t p0 = tile * P + (uint64_t)tid * E;
  float ae[E], ph[E], cs[E], sn[E];
  load_anchors<E>(a_s, p0, n, a_s[n - 1], vec, ae);
  load_anchors<E>(phs, p0, n, 0.f, true, ph);
#pragma unroll
  for (int e = 0; e < E; ++e) sincosf(ph[e], &sn[e], &cs[e]);
  const float2 ta = tanch[tile];
  const float sf = tile > 0 ? tanch[tile - 1].y : ta.x;
  const float sb = tile + 1 < T ? tanch[tile + 1].x : ta.y;
  float acc[E], acc0[E], dph[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = acc0[e] = dph[e] = 0.f;
  static_assert(C == 1, "one input column per pass");
  __shared__ float s_x[kStageCols * P], s_g[kStageCols * P], s_dx[kStageCols * P];
  const uint64_t lo = tile * P;
  const bool vec4 = (m % 4 == 0) && (reinterpret_cast<uintptr_t>(xs) % 16 == 0) && (reinterpret_cast<uintptr_t>(gs) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(dxs) % 16 == 0);
  for (uint32_t cc = 0; cc < m; ++cc) {
    const uint32_t j0 = cc % kStageCols;
    if (j0 == 0) {  // the next slice of columns, loaded once for the whole tile
      const uint32_t w = std::min<uint32_t>(kStageCols, m - cc);
      __syncthreads();
      stage_cols<P, BLOCK>(xs, lo, n, m, cc, w, vec4, s_x);
      stage_cols<P, BLOCK>(gs, lo, n, m, cc, w, vec4, s_g);
      __syncthreads();
    }
    float xv[E][C], gv[E][C], v[E][CC];
    staged_rows<E, P>(s_x, j0, (uint32_t)tid * E, xv);
    staged_rows<E, P>(s_g, j0, (uint32_t)tid * E, gv);
    phased_quad<E, C>(cs, sn, xv, gv, v);
    {
      // both decays in one scan of [v | v]: the tie half first (F0, U0),
      // then the kernel's
      float v2[E][2 * CC], c2f[2 * CC], c2b[2 * CC];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < CC; ++j) v2[e][j] = v2[e][CC + j] = v[e][j];
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        c2f[j] = cfw[tile * M + pbwdcol<C>(m, cc, CC + j)];
        c2b[j] = cbw[tile * M + pbwdcol<C>(m, cc, CC + j)];
        c2f[CC + j] = cfw[tile * M + pbwdcol<C>(m, cc, j)];
        c2b[CC + j] = cbw[tile * M + pbwdcol<C>(m, cc, j)];
      }
      float F2[E][2 * CC], U2[E][2 * CC];
      tile_scan_fu_mix<E, 2 * CC, NW, CC>(ae, v2, c2f, sf, c2b, sb, s_wf, s_wfs, s_wb, s_wbs, F2, U2);
      float dx[E][C];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          {
            const float scx = F2[e][j] - U2[e][j], ssx = F2[e][C + j] - U2[e][C + j];
            const float scg = F2[e][2 * C + j] - U2[e][2 * C + j], ssg = F2[e][3 * C + j] - U2[e][3 * C + j];
            acc0[e] = fmaf(gv[e][j], fmaf(cs[e], scx, sn[e] * ssx), acc0[e]);
            acc0[e] = fmaf(xv[e][j], fmaf(cs[e], scg, sn[e] * ssg), acc0[e]);
          }
          const float(&F)[2 * CC] = F2[e];  // the kernel's half starts at column CC
          const float(&U)[2 * CC] = U2[e];
          constexpr int o = CC;
          const float scx = F[o + j] - U[o + j], ssx = F[o + C + j] - U[o + C + j];
          const float scg = F[o + 2 * C + j] - U[o + 2 * C + j], ssg = F[o + 3 * C + j] - U[o + 3 * C + j];
          acc[e] = fmaf(gv[e][j], fmaf(cs[e], scx, sn[e] * ssx), acc[e]);
          acc[e] = fmaf(xv[e][j], fmaf(cs[e], scg, sn[e] * ssg), acc[e]);
          const float kcx = F[o + j] + U[o + j], ksx = F[o + C + j] + U[o + C + j];
          const float kcg = F[o + 2 * C + j] + U[o + 2 * C + j], ksg = F[o + 3 * C + j] + U[o + 3 * C + j];
          dph[e] = fmaf(-gv[e][j], fmaf(sn[e], kcx, -cs[e] * ksx), dph[e]);
          dph[e] = fmaf(xv[e][j], fmaf(cs[e], ksg, -sn[e] * kcg), dph[e]);
          dx[e][j] = fmaf(cs[e], kcg, sn[e] * ksg);
        }
#pragma unroll
      for (int e = 0; e < E; ++e) s_dx[j0 * P + (uint32_t)tid * E + e] = dx[e][0];
    }
    __syncthreads();
    const uint32_t w = std::min<uint32_t>(kStageCols, m - (cc - j0));
    if (j0 + 1 == w)  // the slice's dx, written back as row pieces
      unstage_cols<P, BLOCK>(dxs, lo, n, m, cc - j0, w, vec4, s_dx);
  }
  float dav[E][1], dpv[E][1];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dav[e][0] = acc0[e] - acc[e];
    dpv[e][0] = dph[e];
  }
  store_rows<E, 1>(das, p0, n, 1, 0, true, dav);
  store_rows<E, 1>(dphs, p0, n, 1, 0, true, dpv);
}

template <int C>
static hipError_t run_pbwd_sym(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm, const SortRoute* route,
                               const float* phi, uint64_t n, uint32_t m, const float* x, const float* g, float* dx, float* da,
                               float* dphi, hipStream_t s) {
  const ApplyWorkspace& w = bw.w;
  constexpr int P = pbwd_block(C) * pbwd_items(C);
  const uint64_t T = (n + P - 1) / P;
  const uint32_t M = 8 * m;
  const dim3 grid((unsigned)T), block(pbwd_block(C));
  const bool routed = route != nullptr && m <= kRouteMaxCols;
  const bool vec = (reinterpret_cast<uintptr_t>(a_s) & 15) == 0;
  hipError_t e;
  if (routed) {
    if ((e = route_forward(*route, n, m, x, w.xs, w.t0, w.t1, s)) != hipSuccess) return e;
    if ((e = route_forward(*route, n, m, g, bw.gs, w.t0, w.t1, s)) != hipSuccess) return e;
    if ((e = route_forward(*route, n, 1, phi, w.phs, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    gather_rows2(x, g, perm, phi, n, m, w.xs, bw.gs, w.phs, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  LAPLEX_LAUNCH("k_pbwd_reduce", n, s,
                k_pbwd_reduce<C><<<grid, block, 0, s>>>(a_s, w.xs, bw.gs, w.phs, n, m, w.bf, w.bb, w.tanch, vec));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tile_carries(w.bf, w.bb, w.tanch, T, M, w.cf, w.cb, w.gbf, w.gbb, w.gcf, w.gcb, w.ganch, s, 4 * m)) != hipSuccess)
    return e;
  LAPLEX_LAUNCH("k_pbwd_apply", n, s,
                k_pbwd_apply<C><<<grid, block, 0, s>>>(a_s, w.xs, bw.gs, w.phs, w.cf, w.cb, w.tanch, n, m, T, w.zs, bw.das,
                                                       bw.dphs, vec));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (routed) {
    if ((e = route_inverse(*route, n, m, w.zs, dx, w.t0, w.t1, s)) != hipSuccess) return e;
    if ((e = route_inverse(*route, n, 1, bw.das, da, w.t0, w.t1, s)) != hipSuccess) return e;
    return route_inverse(*route, n, 1, bw.dphs, dphi, w.t0, w.t1, s);
  }
  scatter_rows3(w.zs, perm, n, m, dx, bw.das, da, bw.dphs, dphi, s);
  return hipGetLastError();
}

// One input column per pass: its 4 scanned columns leave a thread 4 elements
// (wider chunks put 8 or 16 scanned columns on 2 or 1 elements per thread and
// ran up to twice as long).
hipError_t backward_phased(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm, const SortRoute* route,
                           const float* phi, uint64_t n, uint32_t m, const float* x, const float* g, float* dx, float* da,
                           float* dphi, hipStream_t s) {
  return run_pbwd_sym<kPbwdChunk>(bw, a_s, perm, route, phi, n, m, x, g, dx, da, dphi, s);
}

// ---------------------------------------------------------------- general (merged a and b)
// Number of a elements among the first d elements of the merge of sorted a
// (length n) and sorted b (length k), b placed first on equal anchors.
__device__ __forceinline__ uint64_t merge_split(const float* a, uint64_t n, const float* b, uint64_t k, uint64_t d) {
  uint64_t lo = d > k ? d - k : 0, hi = std::min(d, n);
  while (lo < hi) {
    const uint64_t mid = (lo + hi) >> 1;
    if (a[mid] < b[d - 1 - mid])
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

template <int C, bool PH>
__global__ __launch_bounds__(apply_block(PH ? 2 * C : C)) void k_gen_reduce(const float* __restrict__ a_s, uint64_t n, const float* __restrict__ b_s,
                                                            uint64_t k, const float* __restrict__ xbs, const float* __restrict__ psis,
                                                            uint32_t m, uint64_t T, float* __restrict__ bf, float* __restrict__ bb,
                                                            float2* __restrict__ tanch, uint2* __restrict__ tsplit) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int E = apply_items(CC);
  constexpr int BLOCK = apply_block(CC);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_red[2 * NW * CC];
  __shared__ uint64_t s_split[4];
  const uint32_t M = PH ? 2 * m : m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t N = n + k;
  const uint64_t d0 = tile * P, d1 = std::min<uint64_t>(N, d0 + P);
  if (tid == 0) {
    s_split[0] = merge_split(a_s, n, b_s, k, d0);
    s_split[1] = d0 - s_split[0];
  } else if (tid == kWave) {
    s_split[2] = merge_split(a_s, n, b_s, k, d1);
    s_split[3] = d1 - s_split[2];
  }
  __syncthreads();
  const uint64_t i0 = s_split[0], j0 = s_split[1], i1 = s_split[2], j1 = s_split[3];
  float s_first = INFINITY, s_last = -INFINITY;
  if (i0 < i1) {
    s_first = a_s[i0];
    s_last = a_s[i1 - 1];
  }
  if (j0 < j1) {
    s_first = fminf(s_first, b_s[j0]);
    s_last = fmaxf(s_last, b_s[j1 - 1]);
  }
  if (tid == 0) {
    tanch[tile] = make_float2(s_first, s_last);
    tsplit[tile] = make_uint2((uint32_t)i0, (uint32_t)j0);
    if (tile + 1 == T) tsplit[T] = make_uint2((uint32_t)n, (uint32_t)k);
  }
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float sf[CC], sb[CC];
#pragma unroll
    for (int j = 0; j < CC; ++j) sf[j] = sb[j] = 0.f;
    for (uint64_t jb = j0 + tid; jb < j1; jb += BLOCK) {
      const float bj = b_s[jb];
      const float wf = decay(bj - s_last), wb = decay(s_first - bj);
      float cs = 1.f, sn = 0.f;
      if (PH) sincosf(psis[jb], &sn, &cs);
      const float* xr = xbs + jb * m + cc * C;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const float xv = xr[j];
        if (PH) {
          const float vc = cs * xv, vs = sn * xv;
          sf[j] = fmaf(wf, vc, sf[j]);
          sf[C + j] = fmaf(wf, vs, sf[C + j]);
          sb[j] = fmaf(wb, vc, sb[j]);
          sb[C + j] = fmaf(wb, vs, sb[C + j]);
        } else {
          sf[j] = fmaf(wf, xv, sf[j]);
          sb[j] = fmaf(wb, xv, sb[j]);
        }
      }
    }
    int writer = 0;
    block_sum2<CC, NW>(sf, sb, s_red, writer);
    if (writer) {
      float tf = 0.f, tb = 0.f;
      for (int w = 0; w < NW; ++w) {
        tf += s_red[(0 * NW + w) * CC + tid];
        tb += s_red[(1 * NW + w) * CC + tid];
      }
      const uint32_t col = sumcol<C, PH>(m, cc, tid);
      bf[tile * M + col] = tf;
      bb[tile * M + col] = tb;
    }
    __syncthreads();
  }
}

// SCATTER: a-side outputs go to y in original order (through perm_a, phases
// phi in original order); otherwise to y in sorted-a order, with phi already
// in sorted-a order.
template <int C, bool PH, bool SCATTER>
__global__ __launch_bounds__(apply_block(PH ? 2 * C : C)) void k_gen_apply(const float* __restrict__ a_s, const uint32_t* __restrict__ perm_a,
                                                           const float* __restrict__ phi, uint64_t n, const float* __restrict__ b_s,
                                                           uint64_t k, const float* __restrict__ xbs, const float* __restrict__ psis,
                                                           uint32_t m, uint64_t T, const float* __restrict__ cfw,
                                                           const float* __restrict__ cbw, const float2* __restrict__ tanch,
                                                           const uint2* __restrict__ tsplit, float* __restrict__ y) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int E = apply_items(CC);
  constexpr int BLOCK = apply_block(CC);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_a[P], s_b[P];
  __shared__ float s_wf[NW * CC], s_wb[NW * CC], s_wfs[NW], s_wbs[NW];
  const uint32_t M = PH ? 2 * m : m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint2 sp0 = tsplit[tile], sp1 = tsplit[tile + 1];
  const uint32_t na = std::min<uint32_t>(sp1.x - sp0.x, P), nb = std::min<uint32_t>(sp1.y - sp0.y, P - na);
  for (uint32_t i = tid; i < na; i += BLOCK) s_a[i] = a_s[(uint64_t)sp0.x + i];
  for (uint32_t i = tid; i < nb; i += BLOCK) s_b[i] = b_s[(uint64_t)sp0.y + i];
  __syncthreads();
  const float s_max = fmaxf(a_s[n - 1], b_s[k - 1]);
  float ae[E];
  int kind[E];  // 0 pad, 1 a (output), 2 b (input)
  uint32_t idx[E], bbefore[E];
  merge_tile_items<E>(s_a, s_b, na, nb, sp0, s_max, ae, kind, idx, bbefore);
  float cs[E], sn[E];
  uint32_t dst[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    cs[e] = 1.f;
    sn[e] = 0.f;
    dst[e] = 0;
    if (kind[e] == 1) {
      dst[e] = SCATTER ? perm_a[idx[e]] : idx[e];
      if ((uint64_t)dst[e] >= n) dst[e] = 0;
      if (PH) sincosf(phi[dst[e]], &sn[e], &cs[e]);
    } else if (kind[e] == 2 && PH) {
      sincosf(psis[idx[e]], &sn[e], &cs[e]);
    }
  }
  const float2 ta = tanch[tile];
  const float sf = tile > 0 ? tanch[tile - 1].y : ta.x;
  const float sb = tile + 1 < T ? tanch[tile + 1].x : ta.y;
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float v[E][CC];
#pragma unroll
    for (int e = 0; e < E; ++e) {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const float xv = (kind[e] == 2) ? xbs[(uint64_t)idx[e] * m + cc * C + j] : 0.f;
        if (PH) {
          v[e][j] = cs[e] * xv;
          v[e][C + j] = sn[e] * xv;
        } else {
          v[e][j] = xv;
        }
      }
    }
    float cin_f[CC], cin_b[CC];
#pragma unroll
    for (int j = 0; j < CC; ++j) {
      const uint32_t col = sumcol<C, PH>(m, cc, j);
      cin_f[j] = cfw[tile * M + col];
      cin_b[j] = cbw[tile * M + col];
    }
    tile_scan<E, CC, NW>(ae, v, cin_f, sf, cin_b, sb, s_wf, s_wfs, s_wb, s_wbs);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (kind[e] == 1) {
        float* yr = y + (uint64_t)dst[e] * m + cc * C;
#pragma unroll
        for (int j = 0; j < C; ++j) yr[j] = PH ? fmaf(cs[e], v[e][j], sn[e] * v[e][C + j]) : v[e][j];
      }
    }
    __syncthreads();
  }
}

template <int C, bool PH>
static hipError_t run_general(const ApplyWorkspace& w, const float* a_s, const uint32_t* perm_a, const SortRoute* route_a,
                              const float* phi, uint64_t n, const float* b_s, const uint32_t* perm_b, const SortRoute* route_b,
                              const float* psi, uint64_t k, uint32_t m, const float* x, float* y, hipStream_t s) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int P = apply_tile(CC);
  const uint64_t T = (n + k + P - 1) / P;
  const uint32_t M = PH ? 2 * m : m;
  const dim3 grid((unsigned)T), block(apply_block(CC));
  hipError_t e;
  // inputs into sorted-b order
  if (route_b != nullptr && m <= kRouteMaxCols) {
    if ((e = route_forward(*route_b, k, m, x, w.xs, w.t0, w.t1, s)) != hipSuccess) return e;
    if (PH && (e = route_forward(*route_b, k, 1, psi, w.phs, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    gather_rows(x, perm_b, PH ? psi : nullptr, k, m, w.xs, w.phs, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  LAPLEX_LAUNCH(PH ? "k_phased_gen_reduce" : "k_gen_reduce", k, s,
                k_gen_reduce<C, PH><<<grid, block, 0, s>>>(a_s, n, b_s, k, w.xs, w.phs, m, T, w.bf, w.bb, w.tanch, w.tsplit));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tile_carries(w.bf, w.bb, w.tanch, T, M, w.cf, w.cb, w.gbf, w.gbb, w.gcf, w.gcb, w.ganch, s)) != hipSuccess) return e;
  if (route_a != nullptr && m <= kRouteMaxCols) {
    const float* phas = nullptr;
    if (PH) {
      if ((e = route_forward(*route_a, n, 1, phi, w.phas, w.t0, w.t1, s)) != hipSuccess) return e;
      phas = w.phas;
    }
    LAPLEX_LAUNCH(PH ? "k_phased_gen_apply_sorted" : "k_gen_apply_sorted", n, s,
                  k_gen_apply<C, PH, false><<<grid, block, 0, s>>>(a_s, perm_a, phas, n, b_s, k, w.xs, w.phs, m, T, w.cf, w.cb,
                                                                   w.tanch, w.tsplit, w.zs));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return route_inverse(*route_a, n, m, w.zs, y, w.t0, w.t1, s);
  }
  LAPLEX_LAUNCH(PH ? "k_phased_gen_apply" : "k_gen_apply", n, s,
                k_gen_apply<C, PH, true><<<grid, block, 0, s>>>(a_s, perm_a, phi, n, b_s, k, w.xs, w.phs, m, T, w.cf, w.cb,
                                                                w.tanch, w.tsplit, y));
  return hipGetLastError();
}

hipError_t apply_general(const ApplyWorkspace& w, Variant var, const float* a_s, const uint32_t* perm_a, const SortRoute* route_a,
                         const float* phi, uint64_t n, const float* b_s, const uint32_t* perm_b, const SortRoute* route_b,
                         const float* psi, uint64_t k, uint32_t m, const float* x, float* y, hipStream_t s) {
  const bool ph = var == Variant::Phased;
#define LAPLEX_GEN(CW)                                                                                                   \
  return ph ? run_general<CW, true>(w, a_s, perm_a, route_a, phi, n, b_s, perm_b, route_b, psi, k, m, x, y, s)          \
            : run_general<CW, false>(w, a_s, perm_a, route_a, phi, n, b_s, perm_b, route_b, psi, k, m, x, y, s)
  switch (ph ? phased_chunk(m) : column_chunk(m)) {
    case 8: LAPLEX_GEN(8);
    case 4: LAPLEX_GEN(4);
    case 2: LAPLEX_GEN(2);
    default: LAPLEX_GEN(1);
  }
#undef LAPLEX_GEN
}


// ---------------------------------------------------------------- general backward
// Backward of y = K(a, b) x with K_ij = exp(-|a_i - b_j|) (rows a, n; columns
// b, k) for the upstream gradient g = dL/dy:
//     dx_j = sum_i K_ij g_i                                  (K^T g),
//     da_i = -sum_c g_ic sum_j sign(a_i - b_j) K_ij x_jc,
//     db_j = -sum_c x_jc sum_i sign(b_j - a_i) K_ij g_ic       (sign(0) = 0).
// All three come from one pass over the merge of sorted a and sorted b (b first
// on equal anchors), with x injected at b elements and g at a elements.  With
// F, U the strict forward / inclusive backward scans and F0, U0 the same under
// the tie decay, S = (F - U) - (F0 - U0) keeps exactly the anchors strictly
// below minus those strictly above, at either kind of element (at an a element
// the tied b's all lie before it, at a b element the tied a's all lie after).
// So at every element A = sum_c g S(x) + x S(g) (one of the two is zero there)
// gives da at a elements and db at b elements, and dx_j = F + U of g at b_j.
// Summary columns (M = 4m) as in the symmetric backward: [0, m) x, [m, 2m) g
// with the kernel's decay, [2m, 4m) the same with the tie decay.
template <int C>
__global__ __launch_bounds__(bwd_block(C)) void k_gbwd_reduce(const float* __restrict__ a_s, uint64_t n,
                                                               const float* __restrict__ b_s, uint64_t k,
                                                               const float* __restrict__ xbs, const float* __restrict__ gas,
                                                               uint32_t m, uint64_t T, float* __restrict__ bf,
                                                               float* __restrict__ bb, float2* __restrict__ tanch,
                                                               uint2* __restrict__ tsplit) {
  constexpr int CC = 4 * C;
  constexpr int BLOCK = bwd_block(C);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * bwd_items(C);
  __shared__ float s_red[2 * NW * CC];
  __shared__ uint64_t s_split[4];
  const uint32_t M = 4 * m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t N = n + k;
  const uint64_t d0 = tile * P, d1 = std::min<uint64_t>(N, d0 + P);
  if (tid == 0) {
    s_split[0] = merge_split(a_s, n, b_s, k, d0);
    s_split[1] = d0 - s_split[0];
  } else if (tid == kWave) {
    s_split[2] = merge_split(a_s, n, b_s, k, d1);
    s_split[3] = d1 - s_split[2];
  }
  __syncthreads();
  const uint64_t i0 = s_split[0], j0 = s_split[1], i1 = s_split[2], j1 = s_split[3];
  float s_first = INFINITY, s_last = -INFINITY;
  if (i0 < i1) {
    s_first = a_s[i0];
    s_last = a_s[i1 - 1];
  }
  if (j0 < j1) {
    s_first = fminf(s_first, b_s[j0]);
    s_last = fmaxf(s_last, b_s[j1 - 1]);
  }
  if (tid == 0) {
    tanch[tile] = make_float2(s_first, s_last);
    tsplit[tile] = make_uint2((uint32_t)i0, (uint32_t)j0);
    if (tile + 1 == T) tsplit[T] = make_uint2((uint32_t)n, (uint32_t)k);
  }
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float sf[CC], sb[CC];
#pragma unroll
    for (int j = 0; j < CC; ++j) sf[j] = sb[j] = 0.f;
    // x at the b elements of the tile: columns [0, C) and [2C, 3C)
    for (uint64_t jb = j0 + tid; jb < j1; jb += BLOCK) {
      const float s = b_s[jb];
      const float wf = decay(s - s_last), wb = decay(s_first - s);
      const float tf = decay_m<true>(s - s_last), tb = decay_m<true>(s_first - s);
      const float* xr = xbs + jb * m + cc * C;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const float v = xr[j];
        sf[j] = fmaf(wf, v, sf[j]);
        sb[j] = fmaf(wb, v, sb[j]);
        sf[2 * C + j] = fmaf(tf, v, sf[2 * C + j]);
        sb[2 * C + j] = fmaf(tb, v, sb[2 * C + j]);
      }
    }
    // g at the a elements: columns [C, 2C) and [3C, 4C)
    for (uint64_t ia = i0 + tid; ia < i1; ia += BLOCK) {
      const float s = a_s[ia];
      const float wf = decay(s - s_last), wb = decay(s_first - s);
      const float tf = decay_m<true>(s - s_last), tb = decay_m<true>(s_first - s);
      const float* gr = gas + ia * m + cc * C;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const float v = gr[j];
        sf[C + j] = fmaf(wf, v, sf[C + j]);
        sb[C + j] = fmaf(wb, v, sb[C + j]);
        sf[3 * C + j] = fmaf(tf, v, sf[3 * C + j]);
        sb[3 * C + j] = fmaf(tb, v, sb[3 * C + j]);
      }
    }
    int writer = 0;
    block_sum2<CC, NW>(sf, sb, s_red, writer);
    if (writer) {
      float f = 0.f, b = 0.f;
      for (int w = 0; w < NW; ++w) {
        f += s_red[(0 * NW + w) * CC + tid];
        b += s_red[(1 * NW + w) * CC + tid];
      }
      const uint32_t col = bwdcol<C>(m, cc, tid);
      bf[tile * M + col] = f;
      bb[tile * M + col] = b;
    }
    __syncthreads();
  }
}

// Merged tile scans -> dx (sorted-b order), da (sorted-a order), db (sorted-b
// order).
template <int C>
__global__ __launch_bounds__(bwd_block(C)) void k_gbwd_apply(const float* __restrict__ a_s, uint64_t n,
                                                              const float* __restrict__ b_s, uint64_t k,
                                                              const float* __restrict__ xbs, const float* __restrict__ gas,
                                                              uint32_t m, uint64_t T, const float* __restrict__ cfw,
                                                              const float* __restrict__ cbw, const float2* __restrict__ tanch,
                                                              const uint2* __restrict__ tsplit, float* __restrict__ dxs,
                                                              float* __restrict__ das, float* __restrict__ dbs) {
  constexpr int CC = 2 * C;  // columns of one scan (x then g)
  constexpr int E = bwd_items(C);
  constexpr int BLOCK = bwd_block(C);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_a[P], s_b[P];
  constexpr int SW = C == 1 ? 2 * CC : CC;  // columns of one wave summary
  __shared__ float s_wf[NW * SW], s_wb[NW * SW], s_wfs[NW], s_wbs[NW];
  const uint32_t M = 4 * m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint2 sp0 = tsplit[tile], sp1 = tsplit[tile + 1];
  const uint32_t na = std::min<uint32_t>(sp1.x - sp0.x, P), nb = std::min<uint32_t>(sp1.y - sp0.y, P - na);
  for (uint32_t i = tid; i < na; i += BLOCK) s_a[i] = a_s[(uint64_t)sp0.x + i];
  for (uint32_t i = tid; i < nb; i += BLOCK) s_b[i] = b_s[(uint64_t)sp0.y + i];
  __syncthreads();
  const float s_max = fmaxf(a_s[n - 1], b_s[k - 1]);
  float ae[E];
  int kind[E];  // 0 pad, 1 a element (g injected, da out), 2 b element (x injected, dx and db out)
  uint32_t idx[E], bbefore[E];
  merge_tile_items<E>(s_a, s_b, na, nb, sp0, s_max, ae, kind, idx, bbefore);
  const float2 ta = tanch[tile];
  const float sf = tile > 0 ? tanch[tile - 1].y : ta.x;
  const float sb = tile + 1 < T ? tanch[tile + 1].x : ta.y;
  float acc[E], acc0[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = acc0[e] = 0.f;
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float v[E][CC];
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < C; ++j) {
        v[e][j] = kind[e] == 2 ? xbs[(uint64_t)idx[e] * m + cc * C + j] : 0.f;
        v[e][C + j] = kind[e] == 1 ? gas[(uint64_t)idx[e] * m + cc * C + j] : 0.f;
      }
    if constexpr (C == 1) {
      // one column: both decays in one scan of [v | v], the tie half first
      float v2[E][2 * CC], c2f[2 * CC], c2b[2 * CC];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < CC; ++j) v2[e][j] = v2[e][CC + j] = v[e][j];
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        c2f[j] = cfw[tile * M + bwdcol<C>(m, cc, CC + j)];
        c2b[j] = cbw[tile * M + bwdcol<C>(m, cc, CC + j)];
        c2f[CC + j] = cfw[tile * M + bwdcol<C>(m, cc, j)];
        c2b[CC + j] = cbw[tile * M + bwdcol<C>(m, cc, j)];
      }
      float F2[E][2 * CC], U2[E][2 * CC];
      tile_scan_fu_mix<E, 2 * CC, NW, CC>(ae, v2, c2f, sf, c2b, sb, s_wf, s_wfs, s_wb, s_wbs, F2, U2);
#pragma unroll
      for (int e = 0; e < E; ++e) {
#pragma unroll
        for (int j = 0; j < C; ++j) {
          acc0[e] = fmaf(v[e][C + j], F2[e][j] - U2[e][j], acc0[e]);
          acc0[e] = fmaf(v[e][j], F2[e][C + j] - U2[e][C + j], acc0[e]);
          acc[e] = fmaf(v[e][C + j], F2[e][CC + j] - U2[e][CC + j], acc[e]);
          acc[e] = fmaf(v[e][j], F2[e][CC + C + j] - U2[e][CC + C + j], acc[e]);
        }
        if (kind[e] == 2) {
          float* dr = dxs + (uint64_t)idx[e] * m + cc * C;
#pragma unroll
          for (int j = 0; j < C; ++j) dr[j] = F2[e][CC + C + j] + U2[e][CC + C + j];
        }
      }
    } else {
      {
        float ct_f[CC], ct_b[CC];
#pragma unroll
        for (int j = 0; j < CC; ++j) {
          ct_f[j] = cfw[tile * M + bwdcol<C>(m, cc, CC + j)];
          ct_b[j] = cbw[tile * M + bwdcol<C>(m, cc, CC + j)];
        }
        float F0[E][CC], U0[E][CC];
        tile_scan_fu<E, CC, NW, true>(ae, v, ct_f, sf, ct_b, sb, s_wf, s_wfs, s_wb, s_wbs, F0, U0);
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int j = 0; j < C; ++j) {
            acc0[e] = fmaf(v[e][C + j], F0[e][j] - U0[e][j], acc0[e]);
            acc0[e] = fmaf(v[e][j], F0[e][C + j] - U0[e][C + j], acc0[e]);
          }
      }
      __syncthreads();  // the second scan reuses the wave summaries
      {
        float ce_f[CC], ce_b[CC];
#pragma unroll
        for (int j = 0; j < CC; ++j) {
          ce_f[j] = cfw[tile * M + bwdcol<C>(m, cc, j)];
          ce_b[j] = cbw[tile * M + bwdcol<C>(m, cc, j)];
        }
        float F[E][CC], U[E][CC];
        tile_scan_fu<E, CC, NW, false>(ae, v, ce_f, sf, ce_b, sb, s_wf, s_wfs, s_wb, s_wbs, F, U);
#pragma unroll
        for (int e = 0; e < E; ++e) {
#pragma unroll
          for (int j = 0; j < C; ++j) {
            acc[e] = fmaf(v[e][C + j], F[e][j] - U[e][j], acc[e]);
            acc[e] = fmaf(v[e][j], F[e][C + j] - U[e][C + j], acc[e]);
          }
          if (kind[e] == 2) {
            float* dr = dxs + (uint64_t)idx[e] * m + cc * C;
#pragma unroll
            for (int j = 0; j < C; ++j) dr[j] = F[e][C + j] + U[e][C + j];
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (kind[e] == 1) das[idx[e]] = acc0[e] - acc[e];
    if (kind[e] == 2) dbs[idx[e]] = acc0[e] - acc[e];
  }
}

template <int C>
static hipError_t run_bwd_general(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm_a,
                                  const SortRoute* route_a, uint64_t n, const float* b_s, const uint32_t* perm_b,
                                  const SortRoute* route_b, uint64_t k, uint32_t m, const float* x, const float* g, float* dx,
                                  float* da, float* db, hipStream_t s) {
  const ApplyWorkspace& w = bw.w;
  constexpr int P = bwd_tile(C);
  const uint64_t T = (n + k + P - 1) / P;
  const uint32_t M = 4 * m;
  const dim3 grid((unsigned)T), block(bwd_block(C));
  const bool routed_a = route_a != nullptr && m <= kRouteMaxCols;
  const bool routed_b = route_b != nullptr && m <= kRouteMaxCols;
  hipError_t e;
  // x into sorted-b order, g into sorted-a order
  if (routed_b) {
    if ((e = route_forward(*route_b, k, m, x, w.xs, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    gather_rows(x, perm_b, nullptr, k, m, w.xs, nullptr, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (routed_a) {
    if ((e = route_forward(*route_a, n, m, g, bw.gs, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    gather_rows(g, perm_a, nullptr, n, m, bw.gs, nullptr, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  LAPLEX_LAUNCH("k_gbwd_reduce", n + k, s,
                k_gbwd_reduce<C><<<grid, block, 0, s>>>(a_s, n, b_s, k, w.xs, bw.gs, m, T, w.bf, w.bb, w.tanch, w.tsplit));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tile_carries(w.bf, w.bb, w.tanch, T, M, w.cf, w.cb, w.gbf, w.gbb, w.gcf, w.gcb, w.ganch, s, 2 * m)) != hipSuccess)
    return e;
  LAPLEX_LAUNCH("k_gbwd_apply", n + k, s,
                k_gbwd_apply<C><<<grid, block, 0, s>>>(a_s, n, b_s, k, w.xs, bw.gs, m, T, w.cf, w.cb, w.tanch, w.tsplit, w.zs,
                                                       bw.das, bw.dbs));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // back to original order: dx and db along b's route, da along a's
  if (routed_b) {
    if ((e = route_inverse(*route_b, k, m, w.zs, dx, w.t0, w.t1, s)) != hipSuccess) return e;
    if ((e = route_inverse(*route_b, k, 1, bw.dbs, db, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    scatter_rows3(w.zs, perm_b, k, m, dx, bw.dbs, db, nullptr, nullptr, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (routed_a) return route_inverse(*route_a, n, 1, bw.das, da, w.t0, w.t1, s);
  scatter_rows(bw.das, perm_a, n, 1, da, s);
  return hipGetLastError();
}

hipError_t backward_general(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm_a, const SortRoute* route_a,
                            uint64_t n, const float* b_s, const uint32_t* perm_b, const SortRoute* route_b, uint64_t k,
                            uint32_t m, const float* x, const float* g, float* dx, float* da, float* db, hipStream_t s) {
#define LAPLEX_GBWD(CW) \
  return run_bwd_general<CW>(bw, a_s, perm_a, route_a, n, b_s, perm_b, route_b, k, m, x, g, dx, da, db, s)
  switch (column_chunk(m)) {
    case 8: LAPLEX_GBWD(8);
    case 4: LAPLEX_GBWD(4);
    case 2: LAPLEX_GBWD(2);
    default: LAPLEX_GBWD(1);
  }
#undef LAPLEX_GBWD
}


// ---------------------------------------------------------------- weighted Gram matrix
// M = A diag(D) A^T, A = LAPLEX(a, b) (n x n; technical summary, section 2.2,
// Gram operators).  For two output anchors lo <= hi every input anchor b_j
// falls below lo, between them, or above hi, and in each region the product
// exp(-|lo - b_j|) exp(-|hi - b_j|) factors as exp(-(hi - lo)) times a term of
// one anchor only:
//     M = exp(-(hi - lo)) [ P(lo) + (C(hi) - C(lo)) + Q(hi) ],
//     P(s) = sum_{b_j <= s} D_j exp(2 (b_j - s)),   C(s) = sum_{b_j <= s} D_j,
//     Q(s) = sum_{b_j > s} D_j exp(-2 (b_j - s)).
// P and Q are the strict forward and the backward scan of the merge of a and b
// (b first on ties) with the anchors doubled and D injected at b; C is a
// float64 prefix sum of D read at each a (its differences would cancel in
// float32).  Every weight is <= 1.  O(n + k) for these families, then the n^2
// entries, each one exp and a few adds: the fill is bound by writing M.

// Float64 exclusive prefix sums (k + 1) of the weights in sorted-b order.
// One workgroup: each thread sums a contiguous run (independent loads, 8 in
// flight), the 1024 run sums are scanned in LDS (a fixed tree, so the result
// is deterministic), and each run is walked again to write its prefixes.
__global__ __launch_bounds__(1024) void k_gram_dprefix(const float* __restrict__ Ds, uint64_t k, double* __restrict__ Cpre) {
  __shared__ double s_part[1024];
  const uint32_t tid = threadIdx.x;
  const uint64_t q = (k + 1023) / 1024;
  const uint64_t j0 = std::min<uint64_t>(k, (uint64_t)tid * q), j1 = std::min<uint64_t>(k, j0 + q);
  double sum = 0.0;
#pragma unroll 8
  for (uint64_t j = j0; j < j1; ++j) sum += (double)Ds[j];
  s_part[tid] = sum;
  __syncthreads();
  for (uint32_t off = 1; off < 1024; off <<= 1) {
    const double v = tid >= off ? s_part[tid - off] : 0.0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  double run = tid > 0 ? s_part[tid - 1] : 0.0;
#pragma unroll 8
  for (uint64_t j = j0; j < j1; ++j) {
    Cpre[j] = run;
    run += (double)Ds[j];
  }
  if (tid == 1023) Cpre[k] = s_part[1023];
}

// Doubled anchors (exact in float32 for |anchor| < 2^127).
__global__ void k_gram_double(const float* __restrict__ a_s, uint64_t n, const float* __restrict__ b_s, uint64_t k,
                              float* __restrict__ a2, float* __restrict__ b2) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n + k; i += stride) {
    if (i < n)
      a2[i] = 2.f * a_s[i];
    else
      b2[i - n] = 2.f * b_s[i - n];
  }
}

// Merged tile scans with the doubled anchors -> per output anchor, in the
// original order of a: the anchor, P, Q and C.
__global__ __launch_bounds__(apply_block(1)) void k_gram_families(const float* __restrict__ a_s, const float* __restrict__ a2,
                                                                  const uint32_t* __restrict__ perm_a, uint64_t n,
                                                                  const float* __restrict__ b2, uint64_t k,
                                                                  const float* __restrict__ Ds, const double* __restrict__ Cpre,
                                                                  uint64_t T, const float* __restrict__ cfw,
                                                                  const float* __restrict__ cbw, const float2* __restrict__ tanch,
                                                                  const uint2* __restrict__ tsplit, float* __restrict__ Ao,
                                                                  float* __restrict__ Po, float* __restrict__ Qo,
                                                                  double* __restrict__ Co) {
  constexpr int E = apply_items(1);
  constexpr int BLOCK = apply_block(1);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_a[P], s_b[P];
  __shared__ float s_wf[NW], s_wb[NW], s_wfs[NW], s_wbs[NW];
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint2 sp0 = tsplit[tile], sp1 = tsplit[tile + 1];
  const uint32_t na = std::min<uint32_t>(sp1.x - sp0.x, P), nb = std::min<uint32_t>(sp1.y - sp0.y, P - na);
  for (uint32_t i = tid; i < na; i += BLOCK) s_a[i] = a2[(uint64_t)sp0.x + i];
  for (uint32_t i = tid; i < nb; i += BLOCK) s_b[i] = b2[(uint64_t)sp0.y + i];
  __syncthreads();
  const float s_max = fmaxf(a2[n - 1], b2[k - 1]);
  float ae[E];
  int kind[E];
  uint32_t idx[E], bbefore[E];
  merge_tile_items<E>(s_a, s_b, na, nb, sp0, s_max, ae, kind, idx, bbefore);
  float v[E][1];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e][0] = kind[e] == 2 ? Ds[idx[e]] : 0.f;
  const float2 ta = tanch[tile];
  const float sf = tile > 0 ? tanch[tile - 1].y : ta.x;
  const float sb = tile + 1 < T ? tanch[tile + 1].x : ta.y;
  const float cin_f[1] = {cfw[tile]}, cin_b[1] = {cbw[tile]};
  float F[E][1], U[E][1];
  tile_scan_fu<E, 1, NW, false>(ae, v, cin_f, sf, cin_b, sb, s_wf, s_wfs, s_wb, s_wbs, F, U);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (kind[e] == 1) {
      const uint32_t dst = perm_a[idx[e]];
      if ((uint64_t)dst < n) {
        Ao[dst] = a_s[idx[e]];
        Po[dst] = F[e][0];
        Qo[dst] = U[e][0];
        Co[dst] = Cpre[bbefore[e]];
      }
    }
  }
}

// Rows [r0, r0 + rc) of M (original order) into M[(p - r0) * ldm + q].  Each
// thread owns 4 consecutive columns for kGramRows rows; the row's families are
// uniform across the workgroup.  Workgroups run along the columns first
// (block b: column block b mod ncb, row group b / ncb), so the workgroups in
// flight together write whole rows, one contiguous stretch of M.  For a pair with equal anchors the lower
// index plays lo, so both orders of a pair compute the same bits (M is
// exactly symmetric).  zero: k == 0, every entry is 0.
constexpr int kGramRows = 16;
constexpr int kGramBlock = 256;
__global__ __launch_bounds__(kGramBlock) void k_gram_fill(const float* __restrict__ Ao, const float* __restrict__ Po,
                                                          const float* __restrict__ Qo, const double* __restrict__ Co,
                                                          uint64_t n, uint64_t r0, uint64_t rc, float* __restrict__ M,
                                                          uint64_t ldm, bool zero) {
  const uint64_t ncb = (n + 4 * kGramBlock - 1) / (4 * kGramBlock);
  const uint64_t q0 = ((uint64_t)(blockIdx.x % ncb) * kGramBlock + threadIdx.x) * 4;
  const uint64_t rb = (uint64_t)(blockIdx.x / ncb) * kGramRows;
  if (q0 >= n) return;  // no barrier below
  float aq[4], pq[4], qq[4];
  double cq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint64_t q = std::min<uint64_t>(q0 + c, n - 1);
    aq[c] = Ao[q];
    pq[c] = Po[q];
    qq[c] = Qo[q];
    cq[c] = Co[q];
  }
  const bool full = q0 + 4 <= n;
  const bool vec = full && (ldm % 4 == 0) && (reinterpret_cast<uintptr_t>(M) % 16 == 0);
  for (int r = 0; r < kGramRows; ++r) {
    const uint64_t rr = rb + r;
    if (rr >= rc) break;
    const uint64_t p = r0 + rr;
    const float ap = Ao[p], pp = Po[p], qp = Qo[p];
    const double cp = Co[p];
    float out[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t q = q0 + c;
      const bool p_lo = (ap < aq[c]) || (ap == aq[c] && p <= q);
      const float w = decay(-fabsf(aq[c] - ap));
      const float plo = p_lo ? pp : pq[c];
      const float qhi = p_lo ? qq[c] : qp;
      const double dc = p_lo ? (cq[c] - cp) : (cp - cq[c]);
      out[c] = zero ? 0.f : w * ((plo + (float)dc) + qhi);
    }
    float* row = M + rr * ldm + q0;
    if (vec) {
      *reinterpret_cast<float4*>(row) = make_float4(out[0], out[1], out[2], out[3]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (q0 + c < n) row[c] = out[c];
    }
  }
}

hipError_t gram_weighted(const GramWorkspace& g, const float* a_s, const uint32_t* perm_a, uint64_t n, const float* b_s,
                         const uint32_t* perm_b, uint64_t k, const float* D, uint64_t r0, uint64_t rc, float* M, uint64_t ldm,
                         hipStream_t s) {
  hipError_t e;
  // the fill in launches of at most 2^30 workgroups (rows of M in chunks)
  auto fill = [&](bool zero) -> hipError_t {
    const uint64_t ncb = (n + 4 * kGramBlock - 1) / (4 * kGramBlock);
    const uint64_t rows_per = std::max<uint64_t>(1, (1ull << 30) / ncb) * kGramRows;
    for (uint64_t lo = 0; lo < rc; lo += rows_per) {
      const uint64_t cnt = std::min(rows_per, rc - lo);
      const unsigned blocks = (unsigned)(((cnt + kGramRows - 1) / kGramRows) * ncb);
      LAPLEX_LAUNCH("k_gram_fill", cnt * n, s,
                    k_gram_fill<<<blocks, kGramBlock, 0, s>>>(g.Ao, g.Po, g.Qo, g.Co, n, r0 + lo, cnt, M + lo * ldm, ldm,
                                                              zero));
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    return hipSuccess;
  };
  if (k == 0) return fill(true);
  const ApplyWorkspace& w = g.w;
  constexpr int P = apply_tile(1);
  const uint64_t T = (n + k + P - 1) / P;
  const dim3 grid((unsigned)T), block(apply_block(1));
  gather_rows(D, perm_b, nullptr, k, 1, g.Ds, nullptr, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  LAPLEX_LAUNCH("k_gram_dprefix", k, s, k_gram_dprefix<<<1, 1024, 0, s>>>(g.Ds, k, g.Cpre));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  LAPLEX_LAUNCH("k_gram_double", n + k, s,
                k_gram_double<<<rows_grid(n + k), 256, 0, s>>>(a_s, n, b_s, k, g.a2, g.b2));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  LAPLEX_LAUNCH("k_gen_reduce", k, s,
                k_gen_reduce<1, false><<<grid, block, 0, s>>>(g.a2, n, g.b2, k, g.Ds, nullptr, 1, T, w.bf, w.bb, w.tanch, w.tsplit));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tile_carries(w.bf, w.bb, w.tanch, T, 1, w.cf, w.cb, w.gbf, w.gbb, w.gcf, w.gcb, w.ganch, s)) != hipSuccess) return e;
  LAPLEX_LAUNCH("k_gram_families", n + k, s,
                k_gram_families<<<grid, block, 0, s>>>(a_s, g.a2, perm_a, n, g.b2, k, g.Ds, g.Cpre, T, w.cf, w.cb, w.tanch,
                                                       w.tsplit, g.Ao, g.Po, g.Qo, g.Co));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return fill(false);
}


// ---------------------------------------------------------------- general phased backward
// Backward of y = LAPLEX(a, phi; b, psi) x (rows a, n; columns b, k) for
// g = dL/dy.  Over the merge of sorted a and b (b first on ties), cos(psi) x
// and sin(psi) x are injected at b elements and cos(phi) g, sin(phi) g at a
// elements; with each element's own phase (c, s) the symmetric phased
// formulas hold at both kinds (x is zero at a elements, g at b elements):
//     at a: da = -sum_c g (c S(cx) + s S(sx)),   dphi = -sum_c g (s K(cx) - c K(sx)),
//     at b: db = -sum_c x (c S(cg) + s S(sg)),   dpsi =  sum_c x (c K(sg) - s K(cg)),
//           dx = c K(cg) + s K(sg),
// with K = F + U and S = (F - U) - (F0 - U0) as in the general backward (all
// tied b's precede a tied a).  One input column per pass; summary columns as
// in the symmetric phased backward (M = 8m).
__global__ __launch_bounds__(pbwd_block(1)) void k_gpbwd_reduce(const float* __restrict__ a_s, uint64_t n,
                                                                const float* __restrict__ b_s, uint64_t k,
                                                                const float* __restrict__ xbs, const float* __restrict__ psis,
                                                                const float* __restrict__ gas, const float* __restrict__ phas,
                                                                uint32_t m, uint64_t T, float* __restrict__ bf,
                                                                float* __restrict__ bb, float2* __restrict__ tanch,
                                                                uint2* __restrict__ tsplit) {
  constexpr int CC = 8;
  constexpr int BLOCK = pbwd_block(1);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * pbwd_items(1);
  __shared__ float s_red[2 * NW * CC];
  __shared__ uint64_t s_split[4];
  const uint32_t M = 8 * m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t d0 = tile * P, d1 = std::min<uint64_t>(n + k, d0 + P);
  if (tid == 0) {
    s_split[0] = merge_split(a_s, n, b_s, k, d0);
    s_split[1] = d0 - s_split[0];
  } else if (tid == kWave) {
    s_split[2] = merge_split(a_s, n, b_s, k, d1);
    s_split[3] = d1 - s_split[2];
  }
  __syncthreads();
  const uint64_t i0 = s_split[0], j0 = s_split[1], i1 = s_split[2], j1 = s_split[3];
  float s_first = INFINITY, s_last = -INFINITY;
  if (i0 < i1) {
    s_first = a_s[i0];
    s_last = a_s[i1 - 1];
  }
  if (j0 < j1) {
    s_first = fminf(s_first, b_s[j0]);
    s_last = fmaxf(s_last, b_s[j1 - 1]);
  }
  if (tid == 0) {
    tanch[tile] = make_float2(s_first, s_last);
    tsplit[tile] = make_uint2((uint32_t)i0, (uint32_t)j0);
    if (tile + 1 == T) tsplit[T] = make_uint2((uint32_t)n, (uint32_t)k);
  }
  for (uint32_t cc = 0; cc < m; ++cc) {
    float sf[CC], sb[CC];
#pragma unroll
    for (int j = 0; j < CC; ++j) sf[j] = sb[j] = 0.f;
    // b elements: cos(psi) x, sin(psi) x (columns 0, 1; tie 4, 5)
    for (uint64_t jb = j0 + tid; jb < j1; jb += BLOCK) {
      const float t = b_s[jb];
      const float wf = decay(t - s_last), wb = decay(s_first - t);
      const float tf = decay_m<true>(t - s_last), tb = decay_m<true>(s_first - t);
      float sn, cs;
      sincosf(psis[jb], &sn, &cs);
      const float xv = xbs[jb * m + cc];
      const float v0 = cs * xv, v1 = sn * xv;
      sf[0] = fmaf(wf, v0, sf[0]);
      sf[1] = fmaf(wf, v1, sf[1]);
      sb[0] = fmaf(wb, v0, sb[0]);
      sb[1] = fmaf(wb, v1, sb[1]);
      sf[4] = fmaf(tf, v0, sf[4]);
      sf[5] = fmaf(tf, v1, sf[5]);
      sb[4] = fmaf(tb, v0, sb[4]);
      sb[5] = fmaf(tb, v1, sb[5]);
    }
    // a elements: cos(phi) g, sin(phi) g (columns 2, 3; tie 6, 7)
    for (uint64_t ia = i0 + tid; ia < i1; ia += BLOCK) {
      const float t = a_s[ia];
      const float wf = decay(t - s_last), wb = decay(s_first - t);
      const float tf = decay_m<true>(t - s_last), tb = decay_m<true>(s_first - t);
      float sn, cs;
      sincosf(phas[ia], &sn, &cs);
      const float gv = gas[ia * m + cc];
      const float v2 = cs * gv, v3 = sn * gv;
      sf[2] = fmaf(wf, v2, sf[2]);
      sf[3] = fmaf(wf, v3, sf[3]);
      sb[2] = fmaf(wb, v2, sb[2]);
      sb[3] = fmaf(wb, v3, sb[3]);
      sf[6] = fmaf(tf, v2, sf[6]);
      sf[7] = fmaf(tf, v3, sf[7]);
      sb[6] = fmaf(tb, v2, sb[6]);
      sb[7] = fmaf(tb, v3, sb[7]);
    }
    int writer = 0;
    block_sum2<CC, NW>(sf, sb, s_red, writer);
    if (writer) {
      float f = 0.f, b = 0.f;
      for (int w = 0; w < NW; ++w) {
        f += s_red[(0 * NW + w) * CC + tid];
        b += s_red[(1 * NW + w) * CC + tid];
      }
      const uint32_t col = pbwdcol<1>(m, cc, tid);
      bf[tile * M + col] = f;
      bb[tile * M + col] = b;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(pbwd_block(1)) void k_gpbwd_apply(const float* __restrict__ a_s, uint64_t n,
                                                               const float* __restrict__ b_s, uint64_t k,
                                                               const float* __restrict__ xbs, const float* __restrict__ psis,
                                                               const float* __restrict__ gas, const float* __restrict__ phas,
                                                               uint32_t m, uint64_t T, const float* __restrict__ cfw,
                                                               const float* __restrict__ cbw, const float2* __restrict__ tanch,
                                                               const uint2* __restrict__ tsplit, float* __restrict__ dxs,
                                                               float* __restrict__ das, float* __restrict__ dphs,
                                                               float* __restrict__ dbs, float* __restrict__ dpsis) {
  constexpr int CC = 4;
  constexpr int E = pbwd_items(1);
  constexpr int BLOCK = pbwd_block(1);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_a[P], s_b[P];
  __shared__ float s_wf[NW * CC], s_wb[NW * CC], s_wfs[NW], s_wbs[NW];
  const uint32_t M = 8 * m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint2 sp0 = tsplit[tile], sp1 = tsplit[tile + 1];
  const uint32_t na = std::min<uint32_t>(sp1.x - sp0.x, P), nb = std::min<uint32_t>(sp1.y - sp0.y, P - na);
  for (uint32_t i = tid; i < na; i += BLOCK) s_a[i] = a_s[(uint64_t)sp0.x + i];
  for (uint32_t i = tid; i < nb; i += BLOCK) s_b[i] = b_s[(uint64_t)sp0.y + i];
  __syncthreads();
  const float s_max = fmaxf(a_s[n - 1], b_s[k - 1]);
  float ae[E];
  int kind[E];
  uint32_t idx[E], bbefore[E];
  merge_tile_items<E>(s_a, s_b, na, nb, sp0, s_max, ae, kind, idx, bbefore);
  float cs[E], sn[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float ph = kind[e] == 1 ? phas[idx[e]] : (kind[e] == 2 ? psis[idx[e]] : 0.f);
    sincosf(ph, &sn[e], &cs[e]);
  }
  const float2 ta = tanch[tile];
  const float sf = tile > 0 ? tanch[tile - 1].y : ta.x;
  const float sb = tile + 1 < T ? tanch[tile + 1].x : ta.y;
  float acc[E], acc0[E], dph[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = acc0[e] = dph[e] = 0.f;
  for (uint32_t cc = 0; cc < m; ++cc) {
    float xv[E][1], gv[E][1], v[E][CC];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      xv[e][0] = kind[e] == 2 ? xbs[(uint64_t)idx[e] * m + cc] : 0.f;
      gv[e][0] = kind[e] == 1 ? gas[(uint64_t)idx[e] * m + cc] : 0.f;
    }
    phased_quad<E, 1>(cs, sn, xv, gv, v);
    {
      float ct_f[CC], ct_b[CC];
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        ct_f[j] = cfw[tile * M + pbwdcol<1>(m, cc, CC + j)];
        ct_b[j] = cbw[tile * M + pbwdcol<1>(m, cc, CC + j)];
      }
      float F0[E][CC], U0[E][CC];
      tile_scan_fu<E, CC, NW, true>(ae, v, ct_f, sf, ct_b, sb, s_wf, s_wfs, s_wb, s_wbs, F0, U0);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        acc0[e] = fmaf(gv[e][0], fmaf(cs[e], F0[e][0] - U0[e][0], sn[e] * (F0[e][1] - U0[e][1])), acc0[e]);
        acc0[e] = fmaf(xv[e][0], fmaf(cs[e], F0[e][2] - U0[e][2], sn[e] * (F0[e][3] - U0[e][3])), acc0[e]);
      }
    }
    __syncthreads();  // the second scan reuses the wave summaries
    {
      float ce_f[CC], ce_b[CC];
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        ce_f[j] = cfw[tile * M + pbwdcol<1>(m, cc, j)];
        ce_b[j] = cbw[tile * M + pbwdcol<1>(m, cc, j)];
      }
      float F[E][CC], U[E][CC];
      tile_scan_fu<E, CC, NW, false>(ae, v, ce_f, sf, ce_b, sb, s_wf, s_wfs, s_wb, s_wbs, F, U);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        acc[e] = fmaf(gv[e][0], fmaf(cs[e], F[e][0] - U[e][0], sn[e] * (F[e][1] - U[e][1])), acc[e]);
        acc[e] = fmaf(xv[e][0], fmaf(cs[e], F[e][2] - U[e][2], sn[e] * (F[e][3] - U[e][3])), acc[e]);
        const float kcx = F[e][0] + U[e][0], ksx = F[e][1] + U[e][1];
        const float kcg = F[e][2] + U[e][2], ksg = F[e][3] + U[e][3];
        dph[e] = fmaf(-gv[e][0], fmaf(sn[e], kcx, -cs[e] * ksx), dph[e]);
        dph[e] = fmaf(xv[e][0], fmaf(cs[e], ksg, -sn[e] * kcg), dph[e]);
        if (kind[e] == 2) dxs[(uint64_t)idx[e] * m + cc] = fmaf(cs[e], kcg, sn[e] * ksg);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (kind[e] == 1) {
      das[idx[e]] = acc0[e] - acc[e];
      dphs[idx[e]] = dph[e];
    } else if (kind[e] == 2) {
      dbs[idx[e]] = acc0[e] - acc[e];
      dpsis[idx[e]] = dph[e];
    }
  }
}

hipError_t backward_phased_general(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm_a,
                                   const SortRoute* route_a, const float* phi, uint64_t n, const float* b_s,
                                   const uint32_t* perm_b, const SortRoute* route_b, const float* psi, uint64_t k, uint32_t m,
                                   const float* x, const float* g, float* dx, float* da, float* db, float* dphi, float* dpsi,
                                   hipStream_t s) {
  const ApplyWorkspace& w = bw.w;
  constexpr int P = pbwd_block(1) * pbwd_items(1);
  const uint64_t T = (n + k + P - 1) / P;
  const uint32_t M = 8 * m;
  const dim3 grid((unsigned)T), block(pbwd_block(1));
  const bool routed_a = route_a != nullptr && m <= kRouteMaxCols;
  const bool routed_b = route_b != nullptr && m <= kRouteMaxCols;
  hipError_t e;
  // x and psi into sorted-b order, g and phi into sorted-a order
  if (routed_b) {
    if ((e = route_forward(*route_b, k, m, x, w.xs, w.t0, w.t1, s)) != hipSuccess) return e;
    if ((e = route_forward(*route_b, k, 1, psi, w.phs, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    gather_rows(x, perm_b, psi, k, m, w.xs, w.phs, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (routed_a) {
    if ((e = route_forward(*route_a, n, m, g, bw.gs, w.t0, w.t1, s)) != hipSuccess) return e;
    if ((e = route_forward(*route_a, n, 1, phi, w.phas, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    gather_rows(g, perm_a, phi, n, m, bw.gs, w.phas, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  LAPLEX_LAUNCH("k_gpbwd_reduce", n + k, s,
                k_gpbwd_reduce<<<grid, block, 0, s>>>(a_s, n, b_s, k, w.xs, w.phs, bw.gs, w.phas, m, T, w.bf, w.bb, w.tanch,
                                                      w.tsplit));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = tile_carries(w.bf, w.bb, w.tanch, T, M, w.cf, w.cb, w.gbf, w.gbb, w.gcf, w.gcb, w.ganch, s, 4 * m)) != hipSuccess)
    return e;
  LAPLEX_LAUNCH("k_gpbwd_apply", n + k, s,
                k_gpbwd_apply<<<grid, block, 0, s>>>(a_s, n, b_s, k, w.xs, w.phs, bw.gs, w.phas, m, T, w.cf, w.cb, w.tanch,
                                                     w.tsplit, w.zs, bw.das, bw.dphs, bw.dbs, bw.dpsis));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // back to original order: dx, db, dpsi along b's route; da, dphi along a's
  if (routed_b) {
    if ((e = route_inverse(*route_b, k, m, w.zs, dx, w.t0, w.t1, s)) != hipSuccess) return e;
    if ((e = route_inverse(*route_b, k, 1, bw.dbs, db, w.t0, w.t1, s)) != hipSuccess) return e;
    if ((e = route_inverse(*route_b, k, 1, bw.dpsis, dpsi, w.t0, w.t1, s)) != hipSuccess) return e;
  } else {
    scatter_rows3(w.zs, perm_b, k, m, dx, bw.dbs, db, bw.dpsis, dpsi, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (routed_a) {
    if ((e = route_inverse(*route_a, n, 1, bw.das, da, w.t0, w.t1, s)) != hipSuccess) return e;
    return route_inverse(*route_a, n, 1, bw.dphs, dphi, w.t0, w.t1, s);
  }
  scatter_rows3(bw.das, perm_a, n, 1, da, bw.dphs, dphi, nullptr, nullptr, s);
  return hipGetLastError();
}

}  // namespace laplex
