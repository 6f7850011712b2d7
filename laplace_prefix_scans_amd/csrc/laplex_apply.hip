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

namespace laplex {

constexpr int kApplyWaves = kApplyBlock / kWave;

// summary/carry column of injected column j of chunk cc (phased: cos part at
// [0, m), sin part at [m, 2m))
template <int C, bool PH>
__device__ __forceinline__ uint32_t sumcol(uint32_t m, uint32_t cc, int j) {
  if (!PH) return cc * C + (uint32_t)j;
  return (j < C) ? cc * C + (uint32_t)j : m + cc * C + (uint32_t)(j - C);
}

// Sum CC values over the block; totals land in out0[col(j)], out1[col(j)].
template <int CC>
__device__ __forceinline__ void block_sum2(float (&a)[CC], float (&b)[CC], float* s_red /* [2][NW][CC] */, int& jcol_valid) {
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  wave_sum<CC>(a);
  wave_sum<CC>(b);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < CC; ++j) {
      s_red[(0 * kApplyWaves + wid) * CC + j] = a[j];
      s_red[(1 * kApplyWaves + wid) * CC + j] = b[j];
    }
  }
  __syncthreads();
  jcol_valid = threadIdx.x < CC;
}

// ---------------------------------------------------------------- tile scan
// In: v[e][j] injections of this thread's E consecutive elements (anchors
// ae[], nondecreasing across the whole tile); carries into the tile from the
// left (cf, anchored at sf) and right (cb, anchored at sb).
// Out: v[e][j] = strict forward value + inclusive backward value.
template <int E, int CC>
__device__ __forceinline__ void tile_scan(const float (&ae)[E], float (&v)[E][CC], const float (&cf)[CC], float sf,
                                          const float (&cb)[CC], float sb, float* s_wf, float* s_wfs, float* s_wb,
                                          float* s_wbs) {
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  float d[E];  // d[e] = exp(ae[e-1] - ae[e]) for e >= 1
#pragma unroll
  for (int e = 1; e < E; ++e) d[e] = decay(ae[e - 1] - ae[e]);

  // thread-local aggregates
  float B[CC], D[CC];
#pragma unroll
  for (int j = 0; j < CC; ++j) {
    B[j] = v[0][j];
    D[j] = v[E - 1][j];
  }
#pragma unroll
  for (int e = 1; e < E; ++e)
#pragma unroll
    for (int j = 0; j < CC; ++j) B[j] = fmaf(d[e], B[j], v[e][j]);
#pragma unroll
  for (int e = E - 2; e >= 0; --e)
#pragma unroll
    for (int j = 0; j < CC; ++j) D[j] = fmaf(d[e + 1], D[j], v[e][j]);

  // wave scans (forward: by last anchor; backward: by first anchor)
  wave_scan_fwd<CC>(B, ae[E - 1]);
  wave_scan_bwd<CC>(D, ae[0]);
  if (lane == kWave - 1) {
#pragma unroll
    for (int j = 0; j < CC; ++j) s_wf[wid * CC + j] = B[j];
    s_wfs[wid] = ae[E - 1];
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < CC; ++j) s_wb[wid * CC + j] = D[j];
    s_wbs[wid] = ae[0];
  }
  // exclusive values from the neighbouring lanes
  float X[CC], Z[CC];
#pragma unroll
  for (int j = 0; j < CC; ++j) {
    X[j] = __shfl_up(B[j], 1);
    Z[j] = __shfl_down(D[j], 1);
  }
  const float sx = __shfl_up(ae[E - 1], 1);
  const float sz = __shfl_down(ae[0], 1);
  __syncthreads();

  // forward carry into the wave: tile carry, then earlier waves
  float cw[CC];
  float sw = sf;
#pragma unroll
  for (int j = 0; j < CC; ++j) cw[j] = cf[j];
  for (int w = 0; w < wid; ++w) {
    const float s2 = s_wfs[w];
    const float g = decay(sw - s2);
#pragma unroll
    for (int j = 0; j < CC; ++j) cw[j] = fmaf(g, cw[j], s_wf[w * CC + j]);
    sw = s2;
  }
  if (lane > 0) {
    const float g = decay(sw - sx);
#pragma unroll
    for (int j = 0; j < CC; ++j) cw[j] = fmaf(g, cw[j], X[j]);
    sw = sx;
  }
  // backward carry into the wave: tile carry, then later waves
  float cz[CC];
  float sz2 = sb;
#pragma unroll
  for (int j = 0; j < CC; ++j) cz[j] = cb[j];
  for (int w = kApplyWaves - 1; w > wid; --w) {
    const float s2 = s_wbs[w];
    const float g = decay(s2 - sz2);
#pragma unroll
    for (int j = 0; j < CC; ++j) cz[j] = fmaf(g, cz[j], s_wb[w * CC + j]);
    sz2 = s2;
  }
  if (lane < kWave - 1) {
    const float g = decay(sz - sz2);
#pragma unroll
    for (int j = 0; j < CC; ++j) cz[j] = fmaf(g, cz[j], Z[j]);
    sz2 = sz;
  }

  // full forward pass: strict lower part of each element
  const float d0 = decay(sw - ae[0]);
  float F[E][CC];
#pragma unroll
  for (int j = 0; j < CC; ++j) {
    float L = cw[j];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      F[e][j] = (e == 0 ? d0 : d[e]) * L;
      L = v[e][j] + F[e][j];
    }
  }
  // full backward pass, combined
  const float dl = decay(ae[E - 1] - sz2);
#pragma unroll
  for (int j = 0; j < CC; ++j) {
    float U = cz[j];
#pragma unroll
    for (int e = E - 1; e >= 0; --e) {
      U = fmaf(e == E - 1 ? dl : d[e + 1], U, v[e][j]);
      v[e][j] = F[e][j] + U;
    }
  }
}

// ---------------------------------------------------------------- carries
constexpr int kCarryBlock = 1024;

// Scan of the tile aggregates into the carry entering each tile from the left
// (cf: value at the previous tile's last element) and from the right (cb:
// value at the next tile's first element).  One workgroup: each thread folds
// a contiguous run of tiles, wave 0 scans the 1024 run aggregates in 16
// rounds, then each thread walks its run again writing carries.
__global__ __launch_bounds__(kCarryBlock) void k_tile_carry(const float* __restrict__ bf, const float* __restrict__ bb,
                                                            const float2* __restrict__ tanch, uint64_t T, uint32_t M,
                                                            float* __restrict__ cf, float* __restrict__ cb) {
  __shared__ float sB[kCarryBlock], sS[kCarryBlock];
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const uint64_t q = (T + kCarryBlock - 1) / kCarryBlock;
  const uint64_t t0 = std::min<uint64_t>(T, (uint64_t)tid * q), t1 = std::min<uint64_t>(T, t0 + q);
  const float s_min = tanch[0].y, s_maxf = tanch[T - 1].x, s_maxl = tanch[T - 1].y;
  for (uint32_t c = 0; c < M; ++c) {
    // ---- forward
    float B = 0.f, s = s_maxl;
    if (t0 < t1) {
      B = bf[t0 * M + c];
      s = tanch[t0].y;
      for (uint64_t t = t0 + 1; t < t1; ++t) {
        const float s2 = tanch[t].y;
        B = fmaf(decay(s - s2), B, bf[t * M + c]);
        s = s2;
      }
    }
    sB[tid] = B;
    sS[tid] = s;
    __syncthreads();
    if (wid == 0) {
      float cB = 0.f, cS = s_min;
      for (int r = 0; r < kCarryBlock / kWave; ++r) {
        const int i = r * kWave + lane;
        float b1[1] = {sB[i]};
        const float s1 = sS[i];
        wave_scan_fwd<1>(b1, s1);
        const float inc = fmaf(decay(cS - s1), cB, b1[0]);
        float ex = __shfl_up(inc, 1), es = __shfl_up(s1, 1);
        if (lane == 0) {
          ex = cB;
          es = cS;
        }
        sB[i] = ex;
        sS[i] = es;
        cB = __shfl(inc, kWave - 1);
        cS = __shfl(s1, kWave - 1);
      }
    }
    __syncthreads();
    if (t0 < t1) {
      float C = sB[tid], sc = sS[tid];
      for (uint64_t t = t0; t < t1; ++t) {
        cf[t * M + c] = C;
        const float s2 = tanch[t].y;
        C = fmaf(decay(sc - s2), C, bf[t * M + c]);
        sc = s2;
      }
    }
    __syncthreads();
    // ---- backward
    B = 0.f;
    s = s_maxf;
    if (t0 < t1) {
      B = bb[(t1 - 1) * M + c];
      s = tanch[t1 - 1].x;
      for (uint64_t t = t1 - 1; t-- > t0;) {
        const float s2 = tanch[t].x;
        B = fmaf(decay(s2 - s), B, bb[t * M + c]);
        s = s2;
      }
    }
    sB[tid] = B;
    sS[tid] = s;
    __syncthreads();
    if (wid == 0) {
      float cB = 0.f, cS = s_maxf;
      for (int r = kCarryBlock / kWave - 1; r >= 0; --r) {
        const int i = r * kWave + lane;
        float b1[1] = {sB[i]};
        const float s1 = sS[i];
        wave_scan_bwd<1>(b1, s1);
        const float inc = fmaf(decay(s1 - cS), cB, b1[0]);
        float ex = __shfl_down(inc, 1), es = __shfl_down(s1, 1);
        if (lane == kWave - 1) {
          ex = cB;
          es = cS;
        }
        sB[i] = ex;
        sS[i] = es;
        cB = __shfl(inc, 0);
        cS = __shfl(s1, 0);
      }
    }
    __syncthreads();
    if (t0 < t1) {
      float C = sB[tid], sc = sS[tid];
      for (uint64_t t = t1; t-- > t0;) {
        cb[t * M + c] = C;
        const float s2 = tanch[t].x;
        C = fmaf(decay(s2 - sc), C, bb[t * M + c]);
        sc = s2;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- symmetric
template <int C, bool PH>
__global__ __launch_bounds__(kApplyBlock) void k_sym_gather_reduce(const float* __restrict__ a_s, const uint32_t* __restrict__ perm,
                                                                   const float* __restrict__ phi, const float* __restrict__ x,
                                                                   uint64_t n, uint32_t m, float* __restrict__ xs,
                                                                   float* __restrict__ phs, float* __restrict__ bf,
                                                                   float* __restrict__ bb, float2* __restrict__ tanch) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int E = apply_items(CC);
  constexpr int P = kApplyBlock * E;
  __shared__ float s_red[2 * kApplyWaves * CC];
  const uint32_t M = PH ? 2 * m : m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t lo = tile * P;
  const uint64_t hi = std::min<uint64_t>(n, lo + P);
  const float s_first = a_s[lo], s_last = a_s[hi - 1];
  if (tid == 0) tanch[tile] = make_float2(s_first, s_last);
  const uint64_t p0 = lo + (uint64_t)tid * E;
  float wf[E], wb[E], cs[E], sn[E];
  uint32_t src[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t p = p0 + e;
    const bool valid = p < n;
    const float ae = valid ? a_s[p] : s_last;
    src[e] = valid ? perm[p] : 0u;
    if ((uint64_t)src[e] >= n) src[e] = 0;  // a handle from the sort is always in range
    wf[e] = valid ? decay(ae - s_last) : 0.f;
    wb[e] = valid ? decay(s_first - ae) : 0.f;
    cs[e] = 1.f;
    sn[e] = 0.f;
    if (PH) {
      const float ph = valid ? phi[src[e]] : 0.f;
      if (valid) phs[p] = ph;
      sincosf(ph, &sn[e], &cs[e]);
    }
  }
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float sf[CC], sb[CC];
#pragma unroll
    for (int j = 0; j < CC; ++j) sf[j] = sb[j] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t p = p0 + e;
      if (p < n) {
        const float* xr = x + (uint64_t)src[e] * m + cc * C;
        float* xo = xs + p * m + cc * C;
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const float xv = xr[j];
          xo[j] = xv;
          if (PH) {
            const float vc = cs[e] * xv, vs = sn[e] * xv;
            sf[j] = fmaf(wf[e], vc, sf[j]);
            sf[C + j] = fmaf(wf[e], vs, sf[C + j]);
            sb[j] = fmaf(wb[e], vc, sb[j]);
            sb[C + j] = fmaf(wb[e], vs, sb[C + j]);
          } else {
            sf[j] = fmaf(wf[e], xv, sf[j]);
            sb[j] = fmaf(wb[e], xv, sb[j]);
          }
        }
      }
    }
    int writer = 0;
    block_sum2<CC>(sf, sb, s_red, writer);
    if (writer) {
      float tf = 0.f, tb = 0.f;
      for (int w = 0; w < kApplyWaves; ++w) {
        tf += s_red[(0 * kApplyWaves + w) * CC + tid];
        tb += s_red[(1 * kApplyWaves + w) * CC + tid];
      }
      const uint32_t col = sumcol<C, PH>(m, cc, tid);
      bf[tile * M + col] = tf;
      bb[tile * M + col] = tb;
    }
    __syncthreads();
  }
}

template <int C, bool PH>
__global__ __launch_bounds__(kApplyBlock) void k_sym_apply(const float* __restrict__ a_s, const uint32_t* __restrict__ perm,
                                                           const float* __restrict__ xs, const float* __restrict__ phs,
                                                           const float* __restrict__ cfw, const float* __restrict__ cbw,
                                                           const float2* __restrict__ tanch, uint64_t n, uint32_t m, uint64_t T,
                                                           float* __restrict__ y) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int E = apply_items(CC);
  constexpr int P = kApplyBlock * E;
  __shared__ float s_wf[kApplyWaves * CC], s_wb[kApplyWaves * CC], s_wfs[kApplyWaves], s_wbs[kApplyWaves];
  const uint32_t M = PH ? 2 * m : m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t p0 = tile * P + (uint64_t)tid * E;
  const float a_max = a_s[n - 1];
  float ae[E], cs[E], sn[E];
  uint32_t dst[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t p = p0 + e;
    const bool valid = p < n;
    ae[e] = valid ? a_s[p] : a_max;
    dst[e] = valid ? perm[p] : 0u;
    if ((uint64_t)dst[e] >= n) dst[e] = 0;
    cs[e] = 1.f;
    sn[e] = 0.f;
    if (PH) sincosf(valid ? phs[p] : 0.f, &sn[e], &cs[e]);
  }
  const float2 ta = tanch[tile];
  const float sf = tile > 0 ? tanch[tile - 1].y : ta.x;
  const float sb = tile + 1 < T ? tanch[tile + 1].x : ta.y;
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float v[E][CC];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t p = p0 + e;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const float xv = (p < n) ? xs[p * m + cc * C + j] : 0.f;
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
    tile_scan<E, CC>(ae, v, cin_f, sf, cin_b, sb, s_wf, s_wfs, s_wb, s_wbs);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (p0 + e < n) {
        float* yr = y + (uint64_t)dst[e] * m + cc * C;
#pragma unroll
        for (int j = 0; j < C; ++j) yr[j] = PH ? fmaf(cs[e], v[e][j], sn[e] * v[e][C + j]) : v[e][j];
      }
    }
    __syncthreads();
  }
}

template <int C, bool PH>
static hipError_t run_sym(const ApplyWorkspace& w, const float* a_s, const uint32_t* perm, const float* phi, uint64_t n,
                          uint32_t m, const float* x, float* y, hipStream_t s) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int P = apply_tile(CC);
  const uint64_t T = (n + P - 1) / P;
  const uint32_t M = PH ? 2 * m : m;
  LAPLEX_LAUNCH(PH ? "k_phased_gather_reduce" : "k_sym_gather_reduce", s,
                k_sym_gather_reduce<C, PH><<<dim3((unsigned)T), dim3(kApplyBlock), 0, s>>>(a_s, perm, phi, x, n, m, w.xs, w.phs,
                                                                                            w.bf, w.bb, w.tanch));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  LAPLEX_LAUNCH("k_tile_carry", s, k_tile_carry<<<1, kCarryBlock, 0, s>>>(w.bf, w.bb, w.tanch, T, M, w.cf, w.cb));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  LAPLEX_LAUNCH(PH ? "k_phased_apply" : "k_sym_apply", s,
                k_sym_apply<C, PH><<<dim3((unsigned)T), dim3(kApplyBlock), 0, s>>>(a_s, perm, w.xs, w.phs, w.cf, w.cb, w.tanch, n,
                                                                                    m, T, y));
  return hipGetLastError();
}

hipError_t apply_sym(const ApplyWorkspace& w, Variant var, const float* a_s, const uint32_t* perm, const float* phi, uint64_t n,
                     uint32_t m, const float* x, float* y, hipStream_t s) {
  const bool ph = var == Variant::Phased;
  switch (column_chunk(m)) {
    case 8: return ph ? run_sym<8, true>(w, a_s, perm, phi, n, m, x, y, s) : run_sym<8, false>(w, a_s, perm, phi, n, m, x, y, s);
    case 4: return ph ? run_sym<4, true>(w, a_s, perm, phi, n, m, x, y, s) : run_sym<4, false>(w, a_s, perm, phi, n, m, x, y, s);
    case 2: return ph ? run_sym<2, true>(w, a_s, perm, phi, n, m, x, y, s) : run_sym<2, false>(w, a_s, perm, phi, n, m, x, y, s);
    default: return ph ? run_sym<1, true>(w, a_s, perm, phi, n, m, x, y, s) : run_sym<1, false>(w, a_s, perm, phi, n, m, x, y, s);
  }
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

__global__ void k_gather_rows(const float* __restrict__ x, const uint32_t* __restrict__ perm, const float* __restrict__ ph,
                              uint64_t rows, uint32_t m, float* __restrict__ xs, float* __restrict__ phs) {
  uint64_t r = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; r < rows; r += stride) {
    uint32_t src = perm[r];
    if ((uint64_t)src >= rows) src = 0;
    for (uint32_t c = 0; c < m; ++c) xs[r * m + c] = x[(uint64_t)src * m + c];
    if (ph) phs[r] = ph[src];
  }
}

template <int C, bool PH>
__global__ __launch_bounds__(kApplyBlock) void k_gen_reduce(const float* __restrict__ a_s, uint64_t n, const float* __restrict__ b_s,
                                                            uint64_t k, const float* __restrict__ xbs, const float* __restrict__ psis,
                                                            uint32_t m, uint64_t T, float* __restrict__ bf, float* __restrict__ bb,
                                                            float2* __restrict__ tanch, uint2* __restrict__ tsplit) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int E = apply_items(CC);
  constexpr int P = kApplyBlock * E;
  __shared__ float s_red[2 * kApplyWaves * CC];
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
    for (uint64_t jb = j0 + tid; jb < j1; jb += kApplyBlock) {
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
    block_sum2<CC>(sf, sb, s_red, writer);
    if (writer) {
      float tf = 0.f, tb = 0.f;
      for (int w = 0; w < kApplyWaves; ++w) {
        tf += s_red[(0 * kApplyWaves + w) * CC + tid];
        tb += s_red[(1 * kApplyWaves + w) * CC + tid];
      }
      const uint32_t col = sumcol<C, PH>(m, cc, tid);
      bf[tile * M + col] = tf;
      bb[tile * M + col] = tb;
    }
    __syncthreads();
  }
}

template <int C, bool PH>
__global__ __launch_bounds__(kApplyBlock) void k_gen_apply(const float* __restrict__ a_s, const uint32_t* __restrict__ perm_a,
                                                           const float* __restrict__ phi, uint64_t n, const float* __restrict__ b_s,
                                                           uint64_t k, const float* __restrict__ xbs, const float* __restrict__ psis,
                                                           uint32_t m, uint64_t T, const float* __restrict__ cfw,
                                                           const float* __restrict__ cbw, const float2* __restrict__ tanch,
                                                           const uint2* __restrict__ tsplit, float* __restrict__ y) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int E = apply_items(CC);
  constexpr int P = kApplyBlock * E;
  __shared__ float s_a[P], s_b[P];
  __shared__ float s_wf[kApplyWaves * CC], s_wb[kApplyWaves * CC], s_wfs[kApplyWaves], s_wbs[kApplyWaves];
  const uint32_t M = PH ? 2 * m : m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint2 sp0 = tsplit[tile], sp1 = tsplit[tile + 1];
  const uint32_t na = std::min<uint32_t>(sp1.x - sp0.x, P), nb = std::min<uint32_t>(sp1.y - sp0.y, P - na);
  for (uint32_t i = tid; i < na; i += kApplyBlock) s_a[i] = a_s[(uint64_t)sp0.x + i];
  for (uint32_t i = tid; i < nb; i += kApplyBlock) s_b[i] = b_s[(uint64_t)sp0.y + i];
  __syncthreads();
  const float s_max = fmaxf(a_s[n - 1], b_s[k - 1]);
  // this thread's E merged elements
  const uint32_t tot = na + nb;
  const uint32_t dd = std::min<uint32_t>(tot, (uint32_t)tid * E);
  uint32_t lo = dd > nb ? dd - nb : 0u, hi = std::min(dd, na);
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (s_a[mid] < s_b[dd - 1 - mid])
      lo = mid + 1;
    else
      hi = mid;
  }
  uint32_t ii = lo, jj = dd - lo;
  float ae[E];
  int kind[E];  // 0 pad, 1 a (output), 2 b (input)
  uint32_t idx[E];
  // serial merge of E elements, written without branches: every per-element
  // value is selected from the same predicate
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool real = (uint32_t)tid * E + e < tot;
    const float va = ii < na ? s_a[ii] : INFINITY;
    const float vb = jj < nb ? s_b[jj] : INFINITY;
    const bool take_b = real && (jj < nb) && (vb <= va);
    const bool take_a = real && !take_b;
    ae[e] = take_b ? vb : (take_a ? va : s_max);
    kind[e] = take_b ? 2 : (take_a ? 1 : 0);
    idx[e] = take_b ? sp0.y + jj : (take_a ? sp0.x + ii : 0u);
    jj += take_b ? 1u : 0u;
    ii += take_a ? 1u : 0u;
  }
  float cs[E], sn[E];
  uint32_t dst[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    cs[e] = 1.f;
    sn[e] = 0.f;
    dst[e] = 0;
    if (kind[e] == 1) {
      dst[e] = perm_a[idx[e]];
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
    tile_scan<E, CC>(ae, v, cin_f, sf, cin_b, sb, s_wf, s_wfs, s_wb, s_wbs);
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
static hipError_t run_general(const ApplyWorkspace& w, const float* a_s, const uint32_t* perm_a, const float* phi, uint64_t n,
                              const float* b_s, const uint32_t* perm_b, const float* psi, uint64_t k, uint32_t m, const float* x,
                              float* y, hipStream_t s) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int P = apply_tile(CC);
  const uint64_t T = (n + k + P - 1) / P;
  const uint32_t M = PH ? 2 * m : m;
  const unsigned gblocks = (unsigned)std::min<uint64_t>((k + 255) / 256, 8192);
  LAPLEX_LAUNCH("k_gather_rows", s, k_gather_rows<<<gblocks, 256, 0, s>>>(x, perm_b, PH ? psi : nullptr, k, m, w.xs, w.phs));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  LAPLEX_LAUNCH(PH ? "k_phased_gen_reduce" : "k_gen_reduce", s,
                k_gen_reduce<C, PH><<<dim3((unsigned)T), dim3(kApplyBlock), 0, s>>>(a_s, n, b_s, k, w.xs, w.phs, m, T, w.bf, w.bb,
                                                                                     w.tanch, w.tsplit));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  LAPLEX_LAUNCH("k_tile_carry", s, k_tile_carry<<<1, kCarryBlock, 0, s>>>(w.bf, w.bb, w.tanch, T, M, w.cf, w.cb));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  LAPLEX_LAUNCH(PH ? "k_phased_gen_apply" : "k_gen_apply", s,
                k_gen_apply<C, PH><<<dim3((unsigned)T), dim3(kApplyBlock), 0, s>>>(a_s, perm_a, phi, n, b_s, k, w.xs, w.phs, m, T,
                                                                                    w.cf, w.cb, w.tanch, w.tsplit, y));
  return hipGetLastError();
}

hipError_t apply_general(const ApplyWorkspace& w, Variant var, const float* a_s, const uint32_t* perm_a, const float* phi,
                         uint64_t n, const float* b_s, const uint32_t* perm_b, const float* psi, uint64_t k, uint32_t m,
                         const float* x, float* y, hipStream_t s) {
  const bool ph = var == Variant::Phased;
#define LAPLEX_GEN(CW)                                                                                  \
  return ph ? run_general<CW, true>(w, a_s, perm_a, phi, n, b_s, perm_b, psi, k, m, x, y, s)          \
            : run_general<CW, false>(w, a_s, perm_a, phi, n, b_s, perm_b, psi, k, m, x, y, s)
  switch (column_chunk(m)) {
    case 8: LAPLEX_GEN(8);
    case 4: LAPLEX_GEN(4);
    case 2: LAPLEX_GEN(2);
    default: LAPLEX_GEN(1);
  }
#undef LAPLEX_GEN
}

}  // namespace laplex
