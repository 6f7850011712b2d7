// Moving payload rows between original and sorted order along the route the
// radix sort recorded.  A forward pass repeats one radix pass's data movement
// for a payload (read in input order, stage in LDS by tile-local sorted
// position, write each digit's run contiguously); an inverse pass undoes it
// (read each digit's run contiguously into LDS, write in input order).  Four
// passes either way replace one random row gather or scatter, whose 4-byte
// accesses the memory system serves far below its streaming rate.
#include "laplex_kernels.hpp"

namespace laplex {

// Digit of every tile-local sorted position, painted from the run starts:
// wave w paints the runs of digits w, w + NW, ... with its 64 lanes.
template <int NW>
__device__ __forceinline__ void paint_digits(const uint16_t* s_start, uint8_t* s_dig) {
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  for (int d = wid; d < 256; d += NW) {
    const uint32_t lo = s_start[d], hi = s_start[d + 1];
    for (uint32_t p = lo + lane; p < hi; p += kWave) s_dig[p] = (uint8_t)d;
  }
}

// The side of a route pass that runs in input order is read or written in
// groups of kGroup consecutive elements per thread (one 8-byte load of their
// positions, W vector loads of their rows when `vec`); the side that runs in
// digit runs moves one element per thread and step, all steps unrolled.
constexpr int kGroup = 4;

template <int W>
__device__ __forceinline__ void ld_group(const float* __restrict__ p, float (&v)[kGroup * W], bool vec) {
  if (vec) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const float4 q = reinterpret_cast<const float4*>(p)[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kGroup * W; ++i) v[i] = p[i];
  }
}
template <int W>
__device__ __forceinline__ void st_group(float* __restrict__ p, const float (&v)[kGroup * W], bool vec) {
  if (vec) {
#pragma unroll
    for (int i = 0; i < W; ++i) reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < kGroup * W; ++i) p[i] = v[i];
  }
}

// The input-order side as rows of W floats: interleaved (row i at p + i W) or,
// with PLANES (W == 2), two separate arrays p[i], p_b[i] forming row i.  vec:
// every array of the side is 16-byte aligned.
template <int W, bool PLANES>
__device__ __forceinline__ void ld_rows(const float* __restrict__ p, const float* __restrict__ p_b, uint64_t i0,
                                        float (&v)[kGroup * W], bool vec) {
  if constexpr (PLANES) {
    static_assert(W == 2, "two planes make rows of two floats");
    float x0[kGroup], x1[kGroup];
    ld_group<1>(p + i0, x0, vec);
    ld_group<1>(p_b + i0, x1, vec);
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      v[2 * g] = x0[g];
      v[2 * g + 1] = x1[g];
    }
  } else {
    ld_group<W>(p + i0 * W, v, vec);
  }
}
template <int W, bool PLANES>
__device__ __forceinline__ void st_rows(float* __restrict__ p, float* __restrict__ p_b, uint64_t i0, const float (&v)[kGroup * W],
                                        bool vec) {
  if constexpr (PLANES) {
    static_assert(W == 2, "two planes make rows of two floats");
    float x0[kGroup], x1[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      x0[g] = v[2 * g];
      x1[g] = v[2 * g + 1];
    }
    st_group<1>(p + i0, x0, vec);
    st_group<1>(p_b + i0, x1, vec);
  } else {
    st_group<W>(p + i0 * W, v, vec);
  }
}
template <int W, bool PLANES>
__device__ __forceinline__ float ld_one(const float* __restrict__ p, const float* __restrict__ p_b, uint64_t i, int c) {
  return PLANES ? (c == 0 ? p[i] : p_b[i]) : p[i * W + c];
}
template <int W, bool PLANES>
__device__ __forceinline__ void st_one(float* __restrict__ p, float* __restrict__ p_b, uint64_t i, int c, float v) {
  if (PLANES)
    (c == 0 ? p : p_b)[i] = v;
  else
    p[i * W + c] = v;
}

// Tile tables into LDS: run starts (clamped to the tile) and run positions.
__device__ __forceinline__ void load_tables(const uint16_t* __restrict__ dstart, const uint32_t* __restrict__ gbase, uint64_t tile,
                                            uint32_t count, uint16_t* s_start, uint32_t* s_gb) {
  const int tid = threadIdx.x;
  if (tid < 256) {
    s_start[tid] = std::min<uint16_t>(dstart[tile * 256 + tid], (uint16_t)count);
    s_gb[tid] = gbase[tile * 256 + tid];
  }
  if (tid == 0) s_start[256] = (uint16_t)count;
}

// vec: `in` (fwd) or `out` (inv), the input-order side, is 16-byte aligned
// (and in_b / out_b with PLANES).
template <int W, bool PLANES, int TILE>
__global__ __launch_bounds__(kRouteBlock) void k_route_fwd(const float* __restrict__ in, const float* __restrict__ in_b,
                                                          float* __restrict__ out,
                                                          const uint16_t* __restrict__ lpos, const uint16_t* __restrict__ dstart,
                                                          const uint32_t* __restrict__ gbase, uint64_t n, bool vec) {
  static_assert(TILE % (kRouteBlock * kGroup) == 0, "whole position groups per thread");
  constexpr int NW = kRouteBlock / kWave;
  constexpr int STEPS = TILE / kRouteBlock;
  constexpr int GSTEPS = TILE / (kRouteBlock * kGroup);
  __shared__ float s_val[TILE * W];
  __shared__ uint8_t s_dig[TILE];
  __shared__ uint16_t s_start[257];
  __shared__ uint32_t s_gb[256];
  const int tid = threadIdx.x;
  uint64_t tile;
  if (!xcd_tile((n + TILE - 1) / TILE, tile)) return;
  const uint64_t base = tile * TILE;
  const uint32_t count = (uint32_t)std::min<uint64_t>(TILE, n - base);
  // input order side: rows to their tile-local sorted position; every load
  // of the thread is issued before the first LDS write
  uint2 lp2[GSTEPS];
  float vv[GSTEPS][kGroup * W];
#pragma unroll
  for (int r = 0; r < GSTEPS; ++r) {
    const uint32_t i0 = (uint32_t)(r * kRouteBlock + tid) * kGroup;
    if (i0 + kGroup <= count) {
      lp2[r] = *reinterpret_cast<const uint2*>(lpos + base + i0);
      ld_rows<W, PLANES>(in, in_b, base + i0, vv[r], vec);
    }
  }
  load_tables(dstart, gbase, tile, count, s_start, s_gb);
#pragma unroll
  for (int r = 0; r < GSTEPS; ++r) {
    const uint32_t i0 = (uint32_t)(r * kRouteBlock + tid) * kGroup;
    if (i0 + kGroup <= count) {
      const uint32_t lp[kGroup] = {lp2[r].x & 0xFFFFu, lp2[r].x >> 16, lp2[r].y & 0xFFFFu, lp2[r].y >> 16};
      const float(&v)[kGroup * W] = vv[r];
#pragma unroll
      for (int g = 0; g < kGroup; ++g)
        if (lp[g] < count) {
#pragma unroll
          for (int c = 0; c < W; ++c) s_val[lp[g] * W + c] = v[g * W + c];
        }
    } else {
      for (uint32_t i = i0; i < count && i < i0 + kGroup; ++i) {
        const uint32_t lp = lpos[base + i];
        if (lp < count) {
#pragma unroll
          for (int c = 0; c < W; ++c) s_val[lp * W + c] = ld_one<W, PLANES>(in, in_b, base + i, c);
        }
      }
    }
  }
  __syncthreads();
  paint_digits<NW>(s_start, s_dig);
  __syncthreads();
  // digit-run side: each run written contiguously
#pragma unroll
  for (int r = 0; r < STEPS; ++r) {
    const uint32_t i = (uint32_t)(r * kRouteBlock + tid);
    if (i < count) {
      const uint32_t o = s_gb[s_dig[i]] + i;
      if ((uint64_t)o < n) {
#pragma unroll
        for (int c = 0; c < W; ++c) out[(uint64_t)o * W + c] = s_val[i * W + c];
      }
    }
  }
}

template <int W, bool PLANES, int TILE>
__global__ __launch_bounds__(kRouteBlock) void k_route_inv(const float* __restrict__ in, float* __restrict__ out,
                                                          float* __restrict__ out_b,
                                                          const uint16_t* __restrict__ lpos, const uint16_t* __restrict__ dstart,
                                                          const uint32_t* __restrict__ gbase, uint64_t n, bool vec) {
  static_assert(TILE % (kRouteBlock * kGroup) == 0, "whole position groups per thread");
  constexpr int NW = kRouteBlock / kWave;
  constexpr int STEPS = TILE / kRouteBlock;
  constexpr int GSTEPS = TILE / (kRouteBlock * kGroup);
  __shared__ float s_val[TILE * W];
  __shared__ uint8_t s_dig[TILE];
  __shared__ uint16_t s_start[257];
  __shared__ uint32_t s_gb[256];
  const int tid = threadIdx.x;
  uint64_t tile;
  if (!xcd_tile((n + TILE - 1) / TILE, tile)) return;
  const uint64_t base = tile * TILE;
  const uint32_t count = (uint32_t)std::min<uint64_t>(TILE, n - base);
  // the input-order side's positions are loaded first, so that their latency
  // overlaps the tables and the run-side reads
  uint2 lp2[GSTEPS];
#pragma unroll
  for (int r = 0; r < GSTEPS; ++r) {
    const uint32_t i0 = (uint32_t)(r * kRouteBlock + tid) * kGroup;
    lp2[r] = i0 + kGroup <= count ? *reinterpret_cast<const uint2*>(lpos + base + i0) : make_uint2(0u, 0u);
  }
  load_tables(dstart, gbase, tile, count, s_start, s_gb);
  __syncthreads();
  paint_digits<NW>(s_start, s_dig);
  __syncthreads();
  // digit-run side: each run read contiguously
#pragma unroll
  for (int r = 0; r < STEPS; ++r) {
    const uint32_t i = (uint32_t)(r * kRouteBlock + tid);
    if (i < count) {
      const uint32_t src = s_gb[s_dig[i]] + i;
      const bool ok = (uint64_t)src < n;
#pragma unroll
      for (int c = 0; c < W; ++c) s_val[i * W + c] = ok ? in[(uint64_t)src * W + c] : 0.f;
    }
  }
  __syncthreads();
  // input order side
#pragma unroll
  for (int r = 0; r < GSTEPS; ++r) {
    const uint32_t i0 = (uint32_t)(r * kRouteBlock + tid) * kGroup;
    if (i0 + kGroup <= count) {
      const uint32_t lp[kGroup] = {lp2[r].x & 0xFFFFu, lp2[r].x >> 16, lp2[r].y & 0xFFFFu, lp2[r].y >> 16};
      float v[kGroup * W];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        const uint32_t q = std::min<uint32_t>(lp[g], count - 1);
#pragma unroll
        for (int c = 0; c < W; ++c) v[g * W + c] = s_val[q * W + c];
      }
      st_rows<W, PLANES>(out, out_b, base + i0, v, vec);
    } else {
      for (uint32_t i = i0; i < count && i < i0 + kGroup; ++i) {
        const uint32_t q = std::min<uint32_t>(lpos[base + i], count - 1);
#pragma unroll
        for (int c = 0; c < W; ++c) st_one<W, PLANES>(out, out_b, base + i, c, s_val[q * W + c]);
      }
    }
  }
}

// Chunk cover of a tile's digit runs, for rows of W floats (W = 1, 2, 4):
// run d covers global rows [G, G + L); the aligned 4-float chunks that overlap
// it are numbered block-locally from cs[d], the first being global chunk
// c0[d] (chunk_run finds the run of a block-local chunk).  L is clipped to
// the array, so no chunk lies wholly past it.
template <int W, int TILE>
struct RunChunks {
  static constexpr int kMax = TILE * W / 4 + 512;  // sum over runs of (L W + 6) / 4
  uint32_t cs[257];
  uint32_t c0[256];
  uint32_t len[256];
  uint32_t wsum[4];
};

// The run of block-local chunk c (cs[d] <= c < cs[d + 1]; empty runs have
// cs[d] == cs[d + 1] and are passed over): a branch-free binary search over
// the 257 prefix entries in LDS.
template <int W, int TILE>
__device__ __forceinline__ uint32_t chunk_run(const RunChunks<W, TILE>& rc, uint32_t c) {
  uint32_t d = 0;
#pragma unroll
  for (uint32_t step = 128; step >= 1; step >>= 1) d = rc.cs[d + step] <= c ? d + step : d;
  return d;
}

// Called by every thread of the block after s_start / s_gb are written (and
// not yet synchronised); ends with a barrier.
template <int W, int NW, int TILE>
__device__ __forceinline__ void build_chunks(RunChunks<W, TILE>& rc, const uint16_t* s_start, const uint32_t* s_gb, uint64_t n) {
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  __syncthreads();
  uint32_t nch = 0, x = 0;
  if (tid < 256) {
    const uint32_t lo = s_start[tid], hi = s_start[tid + 1];
    const uint64_t G = (uint64_t)(uint32_t)(s_gb[tid] + lo);
    uint64_t L = hi > lo ? hi - lo : 0;
    if (G >= n) L = 0;
    else if (G + L > n) L = n - G;
    const uint64_t c0 = G * W / 4, c1 = ((G + L) * W + 3) / 4;
    nch = L ? (uint32_t)(c1 - c0) : 0u;
    rc.c0[tid] = (uint32_t)c0;
    rc.len[tid] = (uint32_t)L;
    x = wave_incl_sum_u32(nch);
    if (lane == kWave - 1) rc.wsum[wid] = x;
  }
  __syncthreads();
  if (tid < 256) {
    uint32_t pre = 0;
    for (int i = 0; i < wid; ++i) pre += rc.wsum[i];
    rc.cs[tid] = pre + x - nch;
    if (tid == 255) rc.cs[256] = pre + x;
  }
  __syncthreads();
}

// Inverse pass whose digit-run side reads 16-byte aligned chunks (W = 1, 2,
// 4 floats per row; `in` 16-byte aligned).  Each run [G, G + L) of global rows
// is covered by the aligned 4-float chunks that overlap it; a thread loads one
// chunk and keeps the floats of the run, so a wave's loads touch whole cache
// lines instead of one dword per lane.  The floats of a boundary chunk that
// lie outside the run belong to neighbouring runs and are discarded; a chunk
// reaching past the end of the array is read float by float.  vec: `out` is
// 16-byte aligned.
template <int W, bool PLANES, int TILE>
__global__ __launch_bounds__(kRouteBlock) __attribute__((amdgpu_waves_per_eu(W == 1 ? 8 : 1))) void k_route_inv_chunked(const float* __restrict__ in, float* __restrict__ out,
                                                                  float* __restrict__ out_b,
                                                                  const uint16_t* __restrict__ lpos,
                                                                  const uint16_t* __restrict__ dstart,
                                                                  const uint32_t* __restrict__ gbase, uint64_t n, bool vec) {
  static_assert(W == 1 || W == 2 || W == 4, "rows must tile a 16-byte chunk");
  static_assert(TILE % (kRouteBlock * kGroup) == 0, "whole position groups per thread");
  constexpr int NW = kRouteBlock / kWave;
  constexpr int GSTEPS = TILE / (kRouteBlock * kGroup);
  constexpr int MAXCH = RunChunks<W, TILE>::kMax;
  constexpr int CSTEPS = (MAXCH + kRouteBlock - 1) / kRouteBlock;
  constexpr int RPC = 4 / W;  // rows per chunk
  __shared__ float s_val[TILE * W];
  __shared__ uint16_t s_start[257];
  __shared__ uint32_t s_gb[256];
  __shared__ RunChunks<W, TILE> rc;
  const int tid = threadIdx.x;
  uint64_t tile;
  if (!xcd_tile((n + TILE - 1) / TILE, tile)) return;
  const uint64_t base = tile * TILE;
  const uint32_t count = (uint32_t)std::min<uint64_t>(TILE, n - base);
  // the input-order side's positions are requested first, so that their
  // latency overlaps the tables and the run-side reads
  uint2 lp2[GSTEPS];
#pragma unroll
  for (int r = 0; r < GSTEPS; ++r) {
    const uint32_t i0 = (uint32_t)(r * kRouteBlock + tid) * kGroup;
    lp2[r] = i0 + kGroup <= count ? *reinterpret_cast<const uint2*>(lpos + base + i0) : make_uint2(0u, 0u);
  }
  load_tables(dstart, gbase, tile, count, s_start, s_gb);
  build_chunks<W, NW, TILE>(rc, s_start, s_gb, n);
  const uint32_t total = rc.cs[256];
  const uint64_t nfl = n * W;  // >= 4 (the host launches this kernel only then)
  // all chunk loads are issued before any is consumed; a chunk that is not
  // loaded whole (past `total`, or reaching past the array) loads chunk 0.
  // Each chunk's run is kept; its global index is formed again afterwards.
  float4 q[CSTEPS];
  uint32_t dr[CSTEPS];
#pragma unroll
  for (int r = 0; r < CSTEPS; ++r) {
    const uint32_t c = (uint32_t)(r * kRouteBlock + tid);
    const uint32_t d = chunk_run(rc, c < total ? c : 0u);
    dr[r] = d;
    const uint32_t g = rc.c0[d] + (c - rc.cs[d]);  // global chunk index (< n W / 4 + 1 <= 2^32)
    const bool whole = c < total && 4 * (uint64_t)g + 4 <= nfl;
    q[r] = reinterpret_cast<const float4*>(in)[whole ? g : 0u];
  }
#pragma unroll
  for (int r = 0; r < CSTEPS; ++r) {
    const uint32_t c = (uint32_t)(r * kRouteBlock + tid);
    if (c < total) {
      const uint32_t d = dr[r];
      const uint64_t g = rc.c0[d] + (c - rc.cs[d]);
      const uint32_t gb = s_gb[d];
      const uint64_t G = (uint64_t)(uint32_t)(gb + s_start[d]);
      const uint64_t Gend = G + rc.len[d];
      float v[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
      if (4 * g + 4 > nfl) {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (4 * g + k < nfl) ? in[4 * g + k] : 0.f;
      }
#pragma unroll
      for (int rr = 0; rr < RPC; ++rr) {
        const uint64_t row = g * RPC + rr;
        if (row >= G && row < Gend) {
          const uint32_t i = (uint32_t)row - gb;  // tile-local sorted position
#pragma unroll
          for (int cc = 0; cc < W; ++cc) s_val[i * W + cc] = v[rr * W + cc];
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < GSTEPS; ++r) {
    const uint32_t i0 = (uint32_t)(r * kRouteBlock + tid) * kGroup;
    if (i0 + kGroup <= count) {
      const uint32_t lp[kGroup] = {lp2[r].x & 0xFFFFu, lp2[r].x >> 16, lp2[r].y & 0xFFFFu, lp2[r].y >> 16};
      float v[kGroup * W];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        const uint32_t q = std::min<uint32_t>(lp[g], count - 1);
#pragma unroll
        for (int c = 0; c < W; ++c) v[g * W + c] = s_val[q * W + c];
      }
      st_rows<W, PLANES>(out, out_b, base + i0, v, vec);
    } else {
      for (uint32_t i = i0; i < count && i < i0 + kGroup; ++i) {
        const uint32_t q = std::min<uint32_t>(lpos[base + i], count - 1);
#pragma unroll
        for (int c = 0; c < W; ++c) st_one<W, PLANES>(out, out_b, base + i, c, s_val[q * W + c]);
      }
    }
  }
}

// ------------------------------------------------------------------ host side
size_t route_bytes(uint64_t n) {
  const uint64_t tiles = sort_tiles_alloc(n);
  auto up = [](uint64_t b) { return (b + 255) & ~uint64_t(255); };
  return (size_t)(4 * (up(2 * n) + up(tiles * 256 * 2) + up(tiles * 256 * 4)));
}

SortRoute carve_route(const void* base, uint64_t n) {
  const uint64_t tiles = sort_tiles_alloc(n);
  auto up = [](uint64_t b) { return (b + 255) & ~uint64_t(255); };
  uintptr_t p = reinterpret_cast<uintptr_t>(base);
  SortRoute r;
  for (int k = 0; k < 4; ++k) {
    r.lpos[k] = reinterpret_cast<uint16_t*>(p);
    p += up(2 * n);
    r.dstart[k] = reinterpret_cast<uint16_t*>(p);
    p += up(tiles * 256 * 2);
    r.gbase[k] = reinterpret_cast<uint32_t*>(p);
    p += up(tiles * 256 * 4);
  }
  return r;
}

// One pass of a route.  in_b (forward) / out_b (inverse), when given, make the
// input-order side two separate arrays forming rows of W = 2 floats.
template <int W, bool PLANES, int TILE>
static hipError_t route_pass_tile(bool fwd, const SortRoute& r, int k, uint64_t n, const float* in, const float* in_b,
                                  float* out, float* out_b, hipStream_t s) {
  // the input-order side: `in` going forward, `out` going back
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = fwd ? (al(in) && (!PLANES || al(in_b))) : (al(out) && (!PLANES || al(out_b)));
  static const char* const kFwd[5] = {"", "k_route_fwd_w1", "k_route_fwd_w2", "k_route_fwd_w3", "k_route_fwd_w4"};
  static const char* const kInv[5] = {"", "k_route_inv_w1", "k_route_inv_w2", "k_route_inv_w3", "k_route_inv_w4"};
  const uint64_t tiles = (n + TILE - 1) / TILE;
  const uint64_t blocks = ((tiles + kXcds - 1) / kXcds) * kXcds;
  if (fwd)
    LAPLEX_LAUNCH(kFwd[W], n, s,
                  k_route_fwd<W, PLANES, TILE><<<dim3((unsigned)blocks), dim3(kRouteBlock), 0, s>>>(
                      in, in_b, out, r.lpos[k], r.dstart[k], r.gbase[k], n, vec));
  else if (W != 3 && al(in) && n * W >= 4)
    LAPLEX_LAUNCH(kInv[W], n, s,
                  k_route_inv_chunked<W == 3 ? 1 : W, PLANES, TILE><<<dim3((unsigned)blocks), dim3(kRouteBlock), 0, s>>>(
                      in, out, out_b, r.lpos[k], r.dstart[k], r.gbase[k], n, vec));
  else
    LAPLEX_LAUNCH(kInv[W], n, s,
                  k_route_inv<W, PLANES, TILE><<<dim3((unsigned)blocks), dim3(kRouteBlock), 0, s>>>(
                      in, out, out_b, r.lpos[k], r.dstart[k], r.gbase[k], n, vec));
  return hipGetLastError();
}
// the route's tiles are the sort's, whose size follows from n
template <int W, bool PLANES>
static hipError_t route_pass(bool fwd, const SortRoute& r, int k, uint64_t n, const float* in, const float* in_b, float* out,
                             float* out_b, hipStream_t s) {
  if (sort_tile(n) == (uint32_t)kSortTileSmall)
    return route_pass_tile<W, PLANES, kSortTileSmall>(fwd, r, k, n, in, in_b, out, out_b, s);
  return route_pass_tile<W, PLANES, kSortTile>(fwd, r, k, n, in, in_b, out, out_b, s);
}

static hipError_t route_pass_w(bool fwd, const SortRoute& r, int k, uint64_t n, uint32_t W, const float* in, float* out,
                               hipStream_t s) {
  switch (W) {
    case 1: return route_pass<1, false>(fwd, r, k, n, in, nullptr, out, nullptr, s);
    case 2: return route_pass<2, false>(fwd, r, k, n, in, nullptr, out, nullptr, s);
    case 3: return route_pass<3, false>(fwd, r, k, n, in, nullptr, out, nullptr, s);
    case 4: return route_pass<4, false>(fwd, r, k, n, in, nullptr, out, nullptr, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t route_forward(const SortRoute& r, uint64_t n, uint32_t W, const float* in, float* out, float* t0, float* t1,
                         hipStream_t s) {
  const float* src[4] = {in, t0, t1, t0};
  float* dst[4] = {t0, t1, t0, out};
  for (int k = 0; k < 4; ++k) {
    hipError_t e = route_pass_w(true, r, k, n, W, src[k], dst[k], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t route_inverse(const SortRoute& r, uint64_t n, uint32_t W, const float* in, float* out, float* t0, float* t1,
                         hipStream_t s) {
  const float* src[4] = {in, t0, t1, t0};
  float* dst[4] = {t0, t1, t0, out};
  for (int i = 0; i < 4; ++i) {
    hipError_t e = route_pass_w(false, r, 3 - i, n, W, src[i], dst[i], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Two arrays of n floats moved together as rows of two (one pass reads each
// route table once for both): original order -> interleaved sorted rows
// (out: n x 2).  t0, t1: scratch of n x 2 floats each.
hipError_t route_forward_pair(const SortRoute& r, uint64_t n, const float* in0, const float* in1, float* out, float* t0,
                              float* t1, hipStream_t s) {
  hipError_t e = route_pass<2, true>(true, r, 0, n, in0, in1, t0, nullptr, s);
  if (e != hipSuccess) return e;
  const float* src[3] = {t0, t1, t0};
  float* dst[3] = {t1, t0, out};
  for (int k = 1; k < 4; ++k)
    if ((e = route_pass<2, false>(true, r, k, n, src[k - 1], nullptr, dst[k - 1], nullptr, s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace laplex
