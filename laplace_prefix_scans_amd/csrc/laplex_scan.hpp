// Device code of the symmetric scan path: the tile scan, the tile-carry
// kernels, the symmetric reduce and apply kernels and the row gather and
// scatter (LAPLEX technical summary, section 2.2 "Exact Scan Algebra").
// Included by laplex_apply.hip, which holds the host-side launches.
#pragma once
#include "laplex_kernels.hpp"

namespace laplex {

// summary/carry column of injected column j of chunk cc (phased: cos part at
// [0, m), sin part at [m, 2m))
template <int C, bool PH>
__device__ __forceinline__ uint32_t sumcol(uint32_t m, uint32_t cc, int j) {
  if (!PH) return cc * C + (uint32_t)j;
  return (j < C) ? cc * C + (uint32_t)j : m + cc * C + (uint32_t)(j - C);
}

// Sum CC values over the block; totals land in out0[col(j)], out1[col(j)].
// Each wave sums the 2 CC values a then b by transposed wave sums of up to
// 32 values (zeros past 2 CC), and one lane per value stores the wave's sum
// in s_red; threads j < CC then add the waves' sums in wave order.
constexpr int pow2_at_least(int x) { return x <= 1 ? 1 : 2 * pow2_at_least((x + 1) / 2); }
constexpr int log2_exact(int x) { return x <= 1 ? 0 : 1 + log2_exact(x / 2); }
template <int CC, int NW>
__device__ __forceinline__ void block_sum2(float (&a)[CC], float (&b)[CC], float* s_red /* [2][NW][CC] */, int& jcol_valid) {
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  constexpr int N = 2 * CC;
  constexpr int G = N <= 32 ? pow2_at_least(N) : 32;  // values per transposed sum
  constexpr int NG = (N + G - 1) / G;
  constexpr int SH = 6 - log2_exact(G);  // the lane holding value i of a group: i << SH
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int q = g * G + i;
      v[i] = q < CC ? a[q] : (q < N ? b[q - CC] : 0.f);
    }
    const float t = wave_sum_t<G>(v);
    const int q = g * G + (lane >> SH);
    if ((lane & ((1 << SH) - 1)) == 0 && q < N) s_red[(q < CC ? wid : NW + wid) * CC + (q < CC ? q : q - CC)] = t;
  }
  __syncthreads();
  jcol_valid = threadIdx.x < CC;
}

// ---------------------------------------------------------------- tile scan
// In: v[e][j] injections of this thread's E consecutive elements (anchors
// ae[], nondecreasing across the whole tile); carries into the tile from the
// left (cf, anchored at sf) and right (cb, anchored at sb).
// Out: F[e][j] the strict forward value (earlier elements only, tied ones
// included), U[e][j] the inclusive backward value.  Columns [0, NT) scan with
// the tie decay (see decay_m), columns [NT, CC) with the kernel's decay, in
// one pass (the anchor differences, wave exchanges and barriers shared).
template <int E, int CC, int NW, int NT>
__device__ __forceinline__ void tile_scan_fu_mix(const float (&ae)[E], const float (&v)[E][CC], const float (&cf)[CC],
                                                 float sf, const float (&cb)[CC], float sb, float* s_wf, float* s_wfs,
                                                 float* s_wb, float* s_wbs, float (&F)[E][CC], float (&Uo)[E][CC]) {
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  // the decay of column j for anchor difference x
  auto dk = [](float x, int j) -> float { return j < NT ? decay_m<true>(x) : decay_m<false>(x); };
  float dt[E], de[E];  // d[e] = exp(ae[e-1] - ae[e]) for e >= 1, tie and kernel
#pragma unroll
  for (int e = 1; e < E; ++e) {
    dt[e] = NT > 0 ? decay_m<true>(ae[e - 1] - ae[e]) : 0.f;
    de[e] = NT < CC ? decay_m<false>(ae[e - 1] - ae[e]) : 0.f;
  }
  auto dcol = [&](int e, int j) -> float { return j < NT ? dt[e] : de[e]; };

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
    for (int j = 0; j < CC; ++j) B[j] = fmaf(dcol(e, j), B[j], v[e][j]);
#pragma unroll
  for (int e = E - 2; e >= 0; --e)
#pragma unroll
    for (int j = 0; j < CC; ++j) D[j] = fmaf(dcol(e + 1, j), D[j], v[e][j]);

  // wave scans (forward: by last anchor; backward: by first anchor)
  wave_scan_fwd_mix<CC, NT>(B, ae[E - 1]);
  wave_scan_bwd_mix<CC, NT>(D, ae[0]);
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

  // Carries into the wave, as direct weighted sums (every weight <= 1):
  // forward, at the last anchor s_ref of the previous wave (the tile carry's
  // anchor for wave 0), the tile carry weighted by exp(sf - s_ref) plus the
  // aggregate of each wave l < wid weighted by exp(s_end(l) - s_ref);
  // backward, mirrored.  With many waves, lane l < wid holds wave l's term
  // and lane kWave-1 the carry's, and lane sums give every lane the same
  // bits.
  static_assert(NW < kWave, "one lane per wave aggregate plus one for the tile carry");
  const float sw = wid > 0 ? s_wfs[wid - 1] : sf;
  const float sz2 = wid < NW - 1 ? s_wbs[wid + 1] : sb;
  float cw[CC], cz[CC];
  if constexpr (NW <= 4) {
    // Few waves: every lane forms the same sums itself, the tile carry first
    // and then the waves in order, from broadcast reads of their aggregates
    // (a wave-uniform loop of at most NW - 1 steps per direction).
    const int wu = __builtin_amdgcn_readfirstlane(wid);
    {
      const float x = sf - sw, y = sz2 - sb;
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        cw[j] = dk(x, j) * cf[j];
        cz[j] = dk(y, j) * cb[j];
      }
    }
    for (int l = 0; l < wu; ++l) {
      const float x = s_wfs[l] - sw;
      const float wt = NT > 0 ? decay_m<true>(x) : 0.f, we = NT < CC ? decay_m<false>(x) : 0.f;
#pragma unroll
      for (int j = 0; j < CC; ++j) cw[j] = fmaf(j < NT ? wt : we, s_wf[l * CC + j], cw[j]);
    }
    for (int l = NW - 1; l > wu; --l) {
      const float x = sz2 - s_wbs[l];
      const float wt = NT > 0 ? decay_m<true>(x) : 0.f, we = NT < CC ? decay_m<false>(x) : 0.f;
#pragma unroll
      for (int j = 0; j < CC; ++j) cz[j] = fmaf(j < NT ? wt : we, s_wb[l * CC + j], cz[j]);
    }
  } else {
    const bool fw = lane < wid, bw = lane > wid && lane < NW;
    const int lf = fw ? lane : 0, lb = bw ? lane : 0;
    const float xf = fw ? s_wfs[lf] - sw : sf - sw;
    const float xb = bw ? sz2 - s_wbs[lb] : sz2 - sb;
    const bool cf_lane = !fw && lane == kWave - 1, cb_lane = !bw && lane == kWave - 1;
#pragma unroll
    for (int j = 0; j < CC; ++j) {
      const float gf = (fw || cf_lane) ? dk(xf, j) : 0.f;
      const float gb = (bw || cb_lane) ? dk(xb, j) : 0.f;
      cw[j] = fw ? gf * s_wf[lf * CC + j] : (cf_lane ? gf * cf[j] : 0.f);
      cz[j] = bw ? gb * s_wb[lb * CC + j] : (cb_lane ? gb * cb[j] : 0.f);
    }
    wave_sum<CC>(cw);
    wave_sum<CC>(cz);
  }
  float swl = sw, szl = sz2;
  if (lane > 0) {
#pragma unroll
    for (int j = 0; j < CC; ++j) cw[j] = fmaf(dk(swl - sx, j), cw[j], X[j]);
    swl = sx;
  }
  if (lane < kWave - 1) {
#pragma unroll
    for (int j = 0; j < CC; ++j) cz[j] = fmaf(dk(sz - szl, j), cz[j], Z[j]);
    szl = sz;
  }

  // full forward pass: strict lower part of each element
#pragma unroll
  for (int j = 0; j < CC; ++j) {
    const float d0 = dk(swl - ae[0], j);
    float L = cw[j];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      F[e][j] = (e == 0 ? d0 : dcol(e, j)) * L;
      L = v[e][j] + F[e][j];
    }
  }
  // full backward pass, combined
#pragma unroll
  for (int j = 0; j < CC; ++j) {
    const float dl = dk(ae[E - 1] - szl, j);
    float U = cz[j];
#pragma unroll
    for (int e = E - 1; e >= 0; --e) {
      U = fmaf(e == E - 1 ? dl : dcol(e + 1, j), U, v[e][j]);
      Uo[e][j] = U;
    }
  }
}
template <int E, int CC, int NW, bool TIE>
__device__ __forceinline__ void tile_scan_fu(const float (&ae)[E], const float (&v)[E][CC], const float (&cf)[CC], float sf,
                                             const float (&cb)[CC], float sb, float* s_wf, float* s_wfs, float* s_wb,
                                             float* s_wbs, float (&F)[E][CC], float (&Uo)[E][CC]) {
  tile_scan_fu_mix<E, CC, NW, TIE ? CC : 0>(ae, v, cf, sf, cb, sb, s_wf, s_wfs, s_wb, s_wbs, F, Uo);
}

// The operator's tile scan: v[e][j] becomes strict forward + inclusive
// backward, i.e. lower + upper - diagonal.
template <int E, int CC, int NW>
__device__ __forceinline__ void tile_scan(const float (&ae)[E], float (&v)[E][CC], const float (&cf)[CC], float sf,
                                          const float (&cb)[CC], float sb, float* s_wf, float* s_wfs, float* s_wb,
                                          float* s_wbs) {
  float F[E][CC], U[E][CC];
  tile_scan_fu<E, CC, NW, false>(ae, v, cf, sf, cb, sb, s_wf, s_wfs, s_wb, s_wbs, F, U);
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int j = 0; j < CC; ++j) v[e][j] = F[e][j] + U[e][j];
}

// ---------------------------------------------------------------- carries
constexpr int kCarryBlock = 1024;
constexpr int kCarryMaxQ = 16;  // tiles per thread of k_tile_carry at the most
constexpr uint64_t kCarryMaxTiles = (uint64_t)kCarryBlock * kCarryMaxQ;

// Scan of the tile aggregates into the carry entering each tile from the left
// (cf: value at the previous tile's last element) and from the right (cb:
// value at the next tile's first element).  One workgroup per column: thread
// i owns the q = ceil(T / kCarryBlock) consecutive tiles from i q, loads them
// all at once and folds them in both directions as direct weighted sums
// (every weight exp(-|s - s_end|) <= 1); the run aggregates are scanned
// across the wave, the waves' totals reach the later (earlier) waves as
// direct weighted sums through LDS, and each thread walks its run once more
// writing both carries.  Q (a power of two) >= q: the loads per thread; T <=
// kCarryBlock * Q (the caller checks).
template <int Q>
__global__ __launch_bounds__(kCarryBlock) void k_tile_carry(const float* __restrict__ bf, const float* __restrict__ bb,
                                                            const float2* __restrict__ tanch, uint64_t T, uint32_t M,
                                                            uint32_t tie_from, float* __restrict__ cf, float* __restrict__ cb) {
  constexpr int NW = kCarryBlock / kWave;
  __shared__ float s_wf[NW], s_wfs[NW], s_wb[NW], s_wbs[NW];
  const uint32_t c = blockIdx.x;
  const bool tie = c >= tie_from;  // columns from tie_from on scan with the tie decay
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const uint64_t q = (T + kCarryBlock - 1) / kCarryBlock;
  const uint64_t t0 = std::min<uint64_t>(T, (uint64_t)tid * q), t1 = std::min<uint64_t>(T, t0 + q);
  const int nt = (int)(t1 - t0);
  const float s_min = tanch[0].y, s_maxf = tanch[T - 1].x, s_maxl = tanch[T - 1].y;

  // ---- this thread's tiles (clamped into range, every load issued at once)
  float af[Q], al[Q], vf[Q], vb[Q];
#pragma unroll
  for (int u = 0; u < Q; ++u) {
    const uint64_t t = std::min<uint64_t>(t0 + (uint64_t)u, T - 1);
    const float2 an = tanch[t];
    af[u] = an.x;
    al[u] = an.y;
    vf[u] = bf[t * M + c];
    vb[u] = bb[t * M + c];
  }
  // ---- fold both directions: (B, s) anchored at the run's last anchor, (D, sd) at its first
  float s = s_maxl, sd = s_maxf;
#pragma unroll
  for (int u = 0; u < Q; ++u)
    if (u + 1 == nt) s = al[u];
  if (nt > 0) sd = af[0];
  float B = 0.f, D = 0.f;
#pragma unroll
  for (int u = 0; u < Q; ++u) {
    if (u < nt) {
      B = fmaf(decay_r(al[u] - s, tie), vf[u], B);
      D = fmaf(decay_r(sd - af[u], tie), vb[u], D);
    }
  }
  // ---- inclusive scans of the runs across the wave
  float b1[1] = {B}, d1[1] = {D};
  if (tie) {
    wave_scan_fwd<1, true>(b1, s);
    wave_scan_bwd<1, true>(d1, sd);
  } else {
    wave_scan_fwd<1, false>(b1, s);
    wave_scan_bwd<1, false>(d1, sd);
  }
  if (lane == kWave - 1) {
    s_wf[wid] = b1[0];
    s_wfs[wid] = s;
  }
  if (lane == 0) {
    s_wb[wid] = d1[0];
    s_wbs[wid] = sd;
  }
  const float X = __shfl_up(b1[0], 1), sx = __shfl_up(s, 1);
  const float Z = __shfl_down(d1[0], 1), sz = __shfl_down(sd, 1);
  __syncthreads();
  // ---- carries into the wave: the earlier (later) waves' totals, lane l
  // holding wave l's term, summed so that every lane has the same bits
  const float sw = wid > 0 ? s_wfs[wid - 1] : s_min;
  const float sz2 = wid < NW - 1 ? s_wbs[wid + 1] : s_maxf;
  float cw[1], cz[1];
  {
    const bool fw = lane < wid, bw = lane > wid && lane < NW;
    const int lf = fw ? lane : 0, lb = bw ? lane : 0;
    cw[0] = fw ? decay_r(s_wfs[lf] - sw, tie) * s_wf[lf] : 0.f;
    cz[0] = bw ? decay_r(sz2 - s_wbs[lb], tie) * s_wb[lb] : 0.f;
    wave_sum<1>(cw);
    wave_sum<1>(cz);
  }
  // ---- exclusive values of this thread's run, then its tiles' carries
  float C = cw[0], sc = sw;
  if (lane > 0) {
    C = fmaf(decay_r(sw - sx, tie), cw[0], X);
    sc = sx;
  }
  float Cb = cz[0], scb = sz2;
  if (lane < kWave - 1) {
    Cb = fmaf(decay_r(sz - sz2, tie), cz[0], Z);
    scb = sz;
  }
#pragma unroll
  for (int u = 0; u < Q; ++u) {
    if (u < nt) {
      cf[(t0 + (uint64_t)u) * M + c] = C;
      C = fmaf(decay_r(sc - al[u], tie), C, vf[u]);
      sc = al[u];
    }
  }
#pragma unroll
  for (int u = Q - 1; u >= 0; --u) {
    if (u < nt) {
      cb[(t0 + (uint64_t)u) * M + c] = Cb;
      Cb = fmaf(decay_r(af[u] - scb, tie), Cb, vb[u]);
      scb = af[u];
    }
  }
}

// Large tile counts: the tiles are grouped by 1024.  k_carry_up folds each
// group into one aggregate per direction (direct weighted sums), k_tile_carry
// scans the group aggregates, and k_carry_down turns each group's carry into
// the carries of its tiles with a block-wide scan (wave shuffles, then the
// waves' totals in order).  All three run one block per (group, column).
constexpr int kCarryGroup = 1024;

__global__ __launch_bounds__(kCarryGroup) void k_carry_up(const float* __restrict__ bf, const float* __restrict__ bb,
                                                          const float2* __restrict__ tanch, uint64_t T, uint32_t M,
                                                          uint32_t tie_from, float* __restrict__ gbf, float* __restrict__ gbb,
                                                          float2* __restrict__ ganch) {
  constexpr int NW = kCarryGroup / kWave;
  __shared__ float s_red[2 * NW];
  const uint64_t g = blockIdx.x;
  const uint32_t c = blockIdx.y;
  const bool tie = c >= tie_from;
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const uint64_t t0 = g * kCarryGroup, t1 = std::min<uint64_t>(T, t0 + kCarryGroup);
  const uint64_t t = t0 + tid;
  const float s_first = tanch[t0].x, s_last = tanch[t1 - 1].y;
  float vf[1] = {0.f}, vb[1] = {0.f};
  if (t < t1) {
    const float2 ta = tanch[t];
    vf[0] = decay_r(ta.y - s_last, tie) * bf[t * M + c];
    vb[0] = decay_r(s_first - ta.x, tie) * bb[t * M + c];
  }
  wave_sum<1>(vf);
  wave_sum<1>(vb);
  if (lane == 0) {
    s_red[wid] = vf[0];
    s_red[NW + wid] = vb[0];
  }
  __syncthreads();
  if (tid == 0) {
    float f = 0.f, b = 0.f;
    for (int w = 0; w < NW; ++w) {
      f += s_red[w];
      b += s_red[NW + w];
    }
    gbf[g * M + c] = f;
    gbb[g * M + c] = b;
    if (c == 0) ganch[g] = make_float2(s_first, s_last);
  }
}

__global__ __launch_bounds__(kCarryGroup) void k_carry_down(const float* __restrict__ bf, const float* __restrict__ bb,
                                                            const float2* __restrict__ tanch, uint64_t T, uint32_t M,
                                                            const float* __restrict__ gcf, const float* __restrict__ gcb,
                                                            const float2* __restrict__ ganch, uint64_t G,
                                                            uint32_t tie_from, float* __restrict__ cf, float* __restrict__ cb) {
  constexpr int NW = kCarryGroup / kWave;
  __shared__ float s_f[NW], s_fs[NW], s_b[NW], s_bs[NW];
  const uint64_t g = blockIdx.x;
  const uint32_t c = blockIdx.y;
  const bool tie = c >= tie_from;
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const uint64_t t0 = g * kCarryGroup, t1 = std::min<uint64_t>(T, t0 + kCarryGroup);
  const uint64_t t = t0 + tid;
  const bool valid = t < t1;
  const float2 last_tile = tanch[t1 - 1];
  const float2 ta = valid ? tanch[t] : last_tile;
  float B[1] = {valid ? bf[t * M + c] : 0.f};
  float D[1] = {valid ? bb[t * M + c] : 0.f};
  // inclusive scans within the wave (forward by last anchors, backward by first)
  if (tie)
        wave_scan_fwd<1, true>(B, ta.y);
      else
        wave_scan_fwd<1, false>(B, ta.y);
  if (tie)
        wave_scan_bwd<1, true>(D, ta.x);
      else
        wave_scan_bwd<1, false>(D, ta.x);
  if (lane == kWave - 1) {
    s_f[wid] = B[0];
    s_fs[wid] = ta.y;
  }
  if (lane == 0) {
    s_b[wid] = D[0];
    s_bs[wid] = ta.x;
  }
  const float X = __shfl_up(B[0], 1), sx = __shfl_up(ta.y, 1);
  const float Z = __shfl_down(D[0], 1), sz = __shfl_down(ta.x, 1);
  __syncthreads();
  // forward: group carry, earlier waves, then earlier lanes of this wave
  float C = gcf[g * M + c];
  float sc = g > 0 ? ganch[g - 1].y : ganch[0].x;
  for (int w = 0; w < wid; ++w) {
    C = fmaf(decay_r(sc - s_fs[w], tie), C, s_f[w]);
    sc = s_fs[w];
  }
  if (lane > 0) {
    C = fmaf(decay_r(sc - sx, tie), C, X);
    sc = sx;
  }
  // backward: group carry, later waves, then later lanes of this wave
  float Cb = gcb[g * M + c];
  float sb = g + 1 < G ? ganch[g + 1].x : ganch[G - 1].y;
  for (int w = NW - 1; w > wid; --w) {
    Cb = fmaf(decay_r(s_bs[w] - sb, tie), Cb, s_b[w]);
    sb = s_bs[w];
  }
  if (lane < kWave - 1) {
    Cb = fmaf(decay_r(sz - sb, tie), Cb, Z);
    sb = sz;
  }
  if (valid) {
    cf[t * M + c] = C;
    cb[t * M + c] = Cb;
  }
}

// ---------------------------------------------------------------- symmetric
// Contiguous loads and stores of N floats; vector instructions when the
// caller knows the address is 16-byte (N % 4 == 0) or 8-byte (N % 2 == 0)
// aligned.
template <int N>
__device__ __forceinline__ void ld_contig(const float* __restrict__ p, float (&v)[N], bool vec) {
  if constexpr (N % 4 == 0) {
    if (vec) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        const float4 q = reinterpret_cast<const float4*>(p)[i];
        v[4 * i] = q.x;
        v[4 * i + 1] = q.y;
        v[4 * i + 2] = q.z;
        v[4 * i + 3] = q.w;
      }
      return;
    }
  } else if constexpr (N % 2 == 0) {
    if (vec) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const float2 q = reinterpret_cast<const float2*>(p)[i];
        v[2 * i] = q.x;
        v[2 * i + 1] = q.y;
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = p[i];
}
template <int N>
__device__ __forceinline__ void st_contig(float* __restrict__ p, const float (&v)[N], bool vec) {
  if constexpr (N % 4 == 0) {
    if (vec) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
      return;
    }
  } else if constexpr (N % 2 == 0) {
    if (vec) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) reinterpret_cast<float2*>(p)[i] = make_float2(v[2 * i], v[2 * i + 1]);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) p[i] = v[i];
}

// Anchors of this thread's E consecutive sorted positions (pad: `pad`).
template <int E>
__device__ __forceinline__ void load_anchors(const float* __restrict__ a_s, uint64_t p0, uint64_t n, float pad, bool vec,
                                             float (&ae)[E]) {
  if (p0 + E <= n) {
    ld_contig<E>(a_s + p0, ae, vec && (E % 4 == 0 || E % 2 == 0));
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) ae[e] = (p0 + e < n) ? a_s[p0 + e] : pad;
  }
}

// Rows p0 .. p0+E-1, columns [cc*C, cc*C + C) of a row-major n x m array;
// rows past n read as zero.  When m == C the thread's E*C floats are
// contiguous and are loaded as one block.
template <int E, int C>
__device__ __forceinline__ void load_rows(const float* __restrict__ x, uint64_t p0, uint64_t n, uint32_t m, uint32_t cc, bool vec,
                                          float (&xv)[E][C]) {
  if (m == C && p0 + E <= n) {
    float flat[E * C];
    ld_contig<E * C>(x + p0 * C, flat, vec);
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < C; ++j) xv[e][j] = flat[e * C + j];
    return;
  }
  if (C % 4 == 0 && vec && m % 4 == 0 && p0 + E <= n) {  // the chunk of each row as 16-byte pieces
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int q = 0; q < C / 4; ++q) {
        const float4 t = *reinterpret_cast<const float4*>(x + (p0 + e) * m + cc * C + 4 * q);
        xv[e][4 * q] = t.x;
        xv[e][4 * q + 1 < C ? 4 * q + 1 : 0] = t.y;
        xv[e][4 * q + 2 < C ? 4 * q + 2 : 0] = t.z;
        xv[e][4 * q + 3 < C ? 4 * q + 3 : 0] = t.w;
      }
    return;
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int j = 0; j < C; ++j) xv[e][j] = (p0 + e < n) ? x[(p0 + e) * m + cc * C + j] : 0.f;
}
template <int E, int C>
__device__ __forceinline__ void store_rows(float* __restrict__ y, uint64_t p0, uint64_t n, uint32_t m, uint32_t cc, bool vec,
                                           const float (&yv)[E][C]) {
  if (m == C && p0 + E <= n) {
    float flat[E * C];
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < C; ++j) flat[e * C + j] = yv[e][j];
    st_contig<E * C>(y + p0 * C, flat, vec);
    return;
  }
  if (C % 4 == 0 && vec && m % 4 == 0 && p0 + E <= n) {  // the chunk of each row as 16-byte pieces
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int q = 0; q < C / 4; ++q)
        *reinterpret_cast<float4*>(y + (p0 + e) * m + cc * C + 4 * q) =
            make_float4(yv[e][4 * q], yv[e][4 * q + 1 < C ? 4 * q + 1 : 0], yv[e][4 * q + 2 < C ? 4 * q + 2 : 0],
                        yv[e][4 * q + 3 < C ? 4 * q + 3 : 0]);
    return;
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (p0 + e < n)
#pragma unroll
      for (int j = 0; j < C; ++j) y[(p0 + e) * m + cc * C + j] = yv[e][j];
}

// Tile aggregates of the inputs in sorted order (xs, and phs for the phased
// operator).  vec: a_s is 16-byte aligned (workspace buffers always are).
template <int C, bool PH>
__global__ __launch_bounds__(apply_block(PH ? 2 * C : C)) void k_sym_reduce(
    const float* __restrict__ a_s, uint64_t n, uint32_t m, const float* __restrict__ xs, const float* __restrict__ phs,
    float* __restrict__ bf, float* __restrict__ bb, float2* __restrict__ tanch, bool vec) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int E = apply_items(CC);
  constexpr int BLOCK = apply_block(CC);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  __shared__ float s_red[2 * NW * CC];
  const uint32_t M = PH ? 2 * m : m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t lo = tile * P;
  const uint64_t hi = std::min<uint64_t>(n, lo + P);
  const float s_first = a_s[lo], s_last = a_s[hi - 1];
  if (tid == 0) tanch[tile] = make_float2(s_first, s_last);
  const uint64_t p0 = lo + (uint64_t)tid * E;
  float ae[E], wf[E], wb[E], cs[E], sn[E];
  load_anchors<E>(a_s, p0, n, s_last, vec, ae);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool valid = p0 + e < n;
    wf[e] = valid ? decay(ae[e] - s_last) : 0.f;
    wb[e] = valid ? decay(s_first - ae[e]) : 0.f;
    cs[e] = 1.f;
    sn[e] = 0.f;
  }
  if (PH) {
    float ph[E];
    load_anchors<E>(phs, p0, n, 0.f, true, ph);
#pragma unroll
    for (int e = 0; e < E; ++e) sincosf(ph[e], &sn[e], &cs[e]);
  }
  // the next column chunk's rows are requested before this chunk is reduced
  float xv_n[E][C];
  load_rows<E, C>(xs, p0, n, m, 0, true, xv_n);
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float xv[E][C];
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < C; ++j) xv[e][j] = xv_n[e][j];
    if (cc + 1 < m / C) load_rows<E, C>(xs, p0, n, m, cc + 1, true, xv_n);
    float sf[CC], sb[CC];
#pragma unroll
    for (int j = 0; j < CC; ++j) sf[j] = sb[j] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const float v = xv[e][j];
        if (PH) {
          const float vc = cs[e] * v, vs = sn[e] * v;
          sf[j] = fmaf(wf[e], vc, sf[j]);
          sf[C + j] = fmaf(wf[e], vs, sf[C + j]);
          sb[j] = fmaf(wb[e], vc, sb[j]);
          sb[C + j] = fmaf(wb[e], vs, sb[C + j]);
        } else {
          sf[j] = fmaf(wf[e], v, sf[j]);
          sb[j] = fmaf(wb[e], v, sb[j]);
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

// Row loads and stores of a thread's E consecutive rows.  FAST: the block's
// rows are all in range, m == C, and the arrays are aligned for vector access.
template <int E, int C, bool FAST>
__device__ __forceinline__ void load_rows_t(const float* __restrict__ x, uint64_t p0, uint64_t n, uint32_t m, uint32_t cc,
                                            float (&xv)[E][C]) {
  if constexpr (FAST) {
    float flat[E * C];
    ld_contig<E * C>(x + p0 * C, flat, true);
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < C; ++j) xv[e][j] = flat[e * C + j];
  } else {
    load_rows<E, C>(x, p0, n, m, cc, true, xv);
  }
}
template <int E, int C, bool FAST>
__device__ __forceinline__ void store_rows_t(float* __restrict__ y, uint64_t p0, uint64_t n, uint32_t m, uint32_t cc,
                                             const float (&yv)[E][C]) {
  if constexpr (FAST) {
    float flat[E * C];
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < C; ++j) flat[e * C + j] = yv[e][j];
    st_contig<E * C>(y + p0 * C, flat, true);
  } else {
    store_rows<E, C>(y, p0, n, m, cc, true, yv);
  }
}

// SCATTER: y rows written to original order through perm; otherwise to
// sorted order (row p of y).
template <int C, bool PH, bool SCATTER, bool FAST>
__device__ __forceinline__ void sym_apply_tile(const float* __restrict__ a_s, const uint32_t* __restrict__ perm,
                                               const float* __restrict__ xs, const float* __restrict__ phs,
                                               const float* __restrict__ cfw, const float* __restrict__ cbw,
                                               const float2* __restrict__ tanch, uint64_t n, uint32_t m, uint64_t T,
                                               float* __restrict__ y, bool vec, float* s_wf, float* s_wb, float* s_wfs,
                                               float* s_wbs) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int E = apply_items(CC);
  constexpr int BLOCK = apply_block(CC);
  constexpr int NW = BLOCK / kWave;
  constexpr int P = BLOCK * E;
  const uint32_t M = PH ? 2 * m : m;
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint64_t p0 = tile * P + (uint64_t)tid * E;
  // the first column chunk's rows and carries are requested before anything
  // else, so that all of the thread's loads are in flight together
  float xv_n[E][C], cinf_n[CC], cinb_n[CC];
  load_rows_t<E, C, FAST>(xs, p0, n, m, 0, xv_n);
#pragma unroll
  for (int j = 0; j < CC; ++j) {
    const uint32_t col = sumcol<C, PH>(m, 0, j);
    cinf_n[j] = cfw[tile * M + col];
    cinb_n[j] = cbw[tile * M + col];
  }
  float ae[E], cs[E], sn[E];
  uint32_t dst[E];
  if constexpr (FAST) {
    ld_contig<E>(a_s + p0, ae, true);
  } else {
    load_anchors<E>(a_s, p0, n, a_s[n - 1], vec, ae);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t p = p0 + e;
    const bool valid = FAST || p < n;
    dst[e] = 0u;
    if (SCATTER) {
      dst[e] = valid ? perm[p] : 0u;
      if ((uint64_t)dst[e] >= n) dst[e] = 0;
    }
    cs[e] = 1.f;
    sn[e] = 0.f;
  }
  if (PH) {
    float ph[E];
    if constexpr (FAST) {
      ld_contig<E>(phs + p0, ph, true);
    } else {
      load_anchors<E>(phs, p0, n, 0.f, true, ph);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) sincosf(ph[e], &sn[e], &cs[e]);
  }
  const float2 ta = tanch[tile];
  const float sf = tile > 0 ? tanch[tile - 1].y : ta.x;
  const float sb = tile + 1 < T ? tanch[tile + 1].x : ta.y;
  // Scattered rows of two chunks (m == 2C, the phased apply's usual case):
  // the first chunk's outputs are held and each row is written whole with
  // the second, so that both halves reach the row's cache line together.
  const bool hold = SCATTER && PH && m == 2 * C;
  float yprev[E][C];
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int j = 0; j < C; ++j) yprev[e][j] = 0.f;
  for (uint32_t cc = 0; cc < m / C; ++cc) {
    float xv[E][C], cin_f[CC], cin_b[CC];
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < C; ++j) xv[e][j] = xv_n[e][j];
#pragma unroll
    for (int j = 0; j < CC; ++j) {
      cin_f[j] = cinf_n[j];
      cin_b[j] = cinb_n[j];
    }
    if (cc + 1 < m / C) {  // next chunk's loads overlap this chunk's scan
      load_rows_t<E, C, FAST>(xs, p0, n, m, cc + 1, xv_n);
#pragma unroll
      for (int j = 0; j < CC; ++j) {
        const uint32_t col = sumcol<C, PH>(m, cc + 1, j);
        cinf_n[j] = cfw[tile * M + col];
        cinb_n[j] = cbw[tile * M + col];
      }
    }
    float v[E][CC];
#pragma unroll
    for (int e = 0; e < E; ++e) {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        if (PH) {
          v[e][j] = cs[e] * xv[e][j];
          v[e][C + j] = sn[e] * xv[e][j];
        } else {
          v[e][j] = xv[e][j];
        }
      }
    }
    tile_scan<E, CC, NW>(ae, v, cin_f, sf, cin_b, sb, s_wf, s_wfs, s_wb, s_wbs);
    float yv[E][C];
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < C; ++j) yv[e][j] = PH ? fmaf(cs[e], v[e][j], sn[e] * v[e][C + j]) : v[e][j];
    if (SCATTER && hold) {
      if (cc == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int j = 0; j < C; ++j) yprev[e][j] = yv[e][j];
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (FAST || p0 + e < n) {
            float* yr = y + (uint64_t)dst[e] * m;
#pragma unroll
            for (int j = 0; j < C; ++j) yr[j] = yprev[e][j];
#pragma unroll
            for (int j = 0; j < C; ++j) yr[C + j] = yv[e][j];
          }
        }
      }
    } else if (SCATTER) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (FAST || p0 + e < n) {
          float* yr = y + (uint64_t)dst[e] * m + cc * C;
#pragma unroll
          for (int j = 0; j < C; ++j) yr[j] = yv[e][j];
        }
      }
    } else {
      store_rows_t<E, C, FAST>(y, p0, n, m, cc, yv);
    }
    __syncthreads();
  }
}

template <int C, bool PH, bool SCATTER>
__global__ __launch_bounds__(apply_block(PH ? 2 * C : C))
__attribute__((amdgpu_waves_per_eu(!PH && C == 1 ? 8 : 1))) void k_sym_apply(
    const float* __restrict__ a_s, const uint32_t* __restrict__ perm, const float* __restrict__ xs,
    const float* __restrict__ phs, const float* __restrict__ cfw, const float* __restrict__ cbw,
    const float2* __restrict__ tanch, uint64_t n, uint32_t m, uint64_t T, float* __restrict__ y, bool vec) {
  constexpr int CC = PH ? 2 * C : C;
  constexpr int NW = apply_block(CC) / kWave;
  constexpr int P = apply_tile(CC);
  __shared__ float s_wf[NW * CC], s_wb[NW * CC], s_wfs[NW], s_wbs[NW];
  if (vec && m == C && ((uint64_t)blockIdx.x + 1) * P <= n)
    sym_apply_tile<C, PH, SCATTER, true>(a_s, perm, xs, phs, cfw, cbw, tanch, n, m, T, y, vec, s_wf, s_wb, s_wfs, s_wbs);
  else
    sym_apply_tile<C, PH, SCATTER, false>(a_s, perm, xs, phs, cfw, cbw, tanch, n, m, T, y, vec, s_wf, s_wb, s_wfs, s_wbs);
}

// Rows of m floats moved by index: pieces of V floats (one vector access
// each), consecutive threads taking consecutive pieces, so a row is read or
// written whole by neighbouring lanes and the sorted-order side is one
// contiguous stream.
template <int V> struct RowPiece;
template <> struct RowPiece<1> { using T = float; };
template <> struct RowPiece<2> { using T = float2; };
template <> struct RowPiece<4> { using T = float4; };

// row and piece of flat piece index i (P pieces per row)
__device__ __forceinline__ uint64_t piece_row(uint64_t i, uint32_t P, uint64_t items) {
  return items < (1ull << 32) ? (uint64_t)((uint32_t)i / P) : i / P;
}

template <int V>
__global__ void k_scatter_rows(const float* __restrict__ src, const uint32_t* __restrict__ perm, uint64_t rows, uint32_t m,
                               float* __restrict__ dst) {
  using T = typename RowPiece<V>::T;
  const uint32_t P = m / V;
  const uint64_t items = rows * P;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < items; i += stride) {
    const uint64_t r = piece_row(i, P, items);
    const uint32_t c = (uint32_t)(i - r * P);
    const uint32_t d = perm[r];
    if ((uint64_t)d >= rows) continue;  // a handle from the sort is always in range
    *reinterpret_cast<T*>(dst + (uint64_t)d * m + (uint64_t)c * V) = *reinterpret_cast<const T*>(src + r * m + (uint64_t)c * V);
  }
}
// dst[perm[r]] = src[r] (rows of m floats) and, when given, d1[perm[r]] =
// s1[r] and d2[perm[r]] = s2[r] (one float per row): arrays that follow the
// same permutation move in one pass, which reads perm once
template <int V>
__global__ void k_scatter_rows3(const float* __restrict__ src, const uint32_t* __restrict__ perm, uint64_t rows, uint32_t m,
                                float* __restrict__ dst, const float* __restrict__ s1, float* __restrict__ d1,
                                const float* __restrict__ s2, float* __restrict__ d2) {
  using T = typename RowPiece<V>::T;
  const uint32_t P = m / V;
  const uint64_t items = rows * P;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < items; i += stride) {
    const uint64_t r = piece_row(i, P, items);
    const uint32_t c = (uint32_t)(i - r * P);
    const uint32_t d = perm[r];
    if ((uint64_t)d >= rows) continue;  // a handle from the sort is always in range
    *reinterpret_cast<T*>(dst + (uint64_t)d * m + (uint64_t)c * V) = *reinterpret_cast<const T*>(src + r * m + (uint64_t)c * V);
    if (c == 0) {
      if (s1) d1[d] = s1[r];
      if (s2) d2[d] = s2[r];
    }
  }
}
// xs[r] = x[perm[r]] (when x is given) and gs[r] = g[perm[r]], rows of m
// floats, and phs[r] = ph[perm[r]] when ph is given: one pass, perm read once
template <int V>
__global__ void k_gather_rows2(const float* __restrict__ x, const float* __restrict__ g, const uint32_t* __restrict__ perm,
                               const float* __restrict__ ph, uint64_t rows, uint32_t m, float* __restrict__ xs,
                               float* __restrict__ gs, float* __restrict__ phs) {
  using T = typename RowPiece<V>::T;
  const uint32_t P = m / V;
  const uint64_t items = rows * P;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < items; i += stride) {
    const uint64_t r = piece_row(i, P, items);
    const uint32_t c = (uint32_t)(i - r * P);
    uint32_t src = perm[r];
    if ((uint64_t)src >= rows) src = 0;
    const uint64_t o = (uint64_t)c * V;
    if (x) *reinterpret_cast<T*>(xs + r * m + o) = *reinterpret_cast<const T*>(x + (uint64_t)src * m + o);
    *reinterpret_cast<T*>(gs + r * m + o) = *reinterpret_cast<const T*>(g + (uint64_t)src * m + o);
    if (ph && c == 0) phs[r] = ph[src];
  }
}
template <int V>
__global__ void k_gather_rows(const float* __restrict__ x, const uint32_t* __restrict__ perm, const float* __restrict__ ph,
                              uint64_t rows, uint32_t m, float* __restrict__ xs, float* __restrict__ phs) {
  using T = typename RowPiece<V>::T;
  const uint32_t P = m / V;
  const uint64_t items = rows * P;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < items; i += stride) {
    const uint64_t r = piece_row(i, P, items);
    const uint32_t c = (uint32_t)(i - r * P);
    uint32_t src = perm[r];
    if ((uint64_t)src >= rows) src = 0;
    *reinterpret_cast<T*>(xs + r * m + (uint64_t)c * V) = *reinterpret_cast<const T*>(x + (uint64_t)src * m + (uint64_t)c * V);
    if (ph && c == 0) phs[r] = ph[src];
  }
}

}  // namespace laplex
