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

template <int W>
__global__ __launch_bounds__(kSortBlock) void k_route_fwd(const float* __restrict__ in, float* __restrict__ out,
                                                          const uint16_t* __restrict__ lpos, const uint16_t* __restrict__ dstart,
                                                          const uint32_t* __restrict__ gbase, uint64_t n) {
  constexpr int TILE = kSortTile;
  constexpr int NW = kSortBlock / kWave;
  __shared__ float s_val[TILE * W];
  __shared__ uint8_t s_dig[TILE];
  __shared__ uint16_t s_start[257];
  __shared__ uint32_t s_gb[256];
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x, base = tile * TILE;
  const uint32_t count = (uint32_t)std::min<uint64_t>(TILE, n - base);
  s_start[tid] = std::min<uint16_t>(dstart[tile * 256 + tid], (uint16_t)count);
  s_gb[tid] = gbase[tile * 256 + tid];
  if (tid == 0) s_start[256] = (uint16_t)count;
  __syncthreads();
  paint_digits<NW>(s_start, s_dig);
  for (uint32_t i = tid; i < count; i += kSortBlock) {
    const uint64_t j = base + i;
    const uint32_t lp = lpos[j];
    if (lp < count) {
#pragma unroll
      for (int c = 0; c < W; ++c) s_val[lp * W + c] = in[j * W + c];
    }
  }
  __syncthreads();
  for (uint32_t i = tid; i < count; i += kSortBlock) {
    const uint32_t o = s_gb[s_dig[i]] + i;
    if ((uint64_t)o < n) {
#pragma unroll
      for (int c = 0; c < W; ++c) out[(uint64_t)o * W + c] = s_val[i * W + c];
    }
  }
}

template <int W>
__global__ __launch_bounds__(kSortBlock) void k_route_inv(const float* __restrict__ in, float* __restrict__ out,
                                                          const uint16_t* __restrict__ lpos, const uint16_t* __restrict__ dstart,
                                                          const uint32_t* __restrict__ gbase, uint64_t n) {
  constexpr int TILE = kSortTile;
  constexpr int NW = kSortBlock / kWave;
  __shared__ float s_val[TILE * W];
  __shared__ uint8_t s_dig[TILE];
  __shared__ uint16_t s_start[257];
  __shared__ uint32_t s_gb[256];
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x, base = tile * TILE;
  const uint32_t count = (uint32_t)std::min<uint64_t>(TILE, n - base);
  s_start[tid] = std::min<uint16_t>(dstart[tile * 256 + tid], (uint16_t)count);
  s_gb[tid] = gbase[tile * 256 + tid];
  if (tid == 0) s_start[256] = (uint16_t)count;
  __syncthreads();
  paint_digits<NW>(s_start, s_dig);
  __syncthreads();
  for (uint32_t i = tid; i < count; i += kSortBlock) {
    const uint32_t src = s_gb[s_dig[i]] + i;
    const bool ok = (uint64_t)src < n;
#pragma unroll
    for (int c = 0; c < W; ++c) s_val[i * W + c] = ok ? in[(uint64_t)src * W + c] : 0.f;
  }
  __syncthreads();
  for (uint32_t i = tid; i < count; i += kSortBlock) {
    const uint64_t j = base + i;
    const uint32_t lp = std::min<uint32_t>(lpos[j], count - 1);
#pragma unroll
    for (int c = 0; c < W; ++c) out[j * W + c] = s_val[lp * W + c];
  }
}

// ------------------------------------------------------------------ host side
size_t route_bytes(uint64_t n) {
  const uint64_t tiles = (n + kSortTile - 1) / kSortTile;
  auto up = [](uint64_t b) { return (b + 255) & ~uint64_t(255); };
  return (size_t)(4 * (up(2 * n) + up(tiles * 256 * 2) + up(tiles * 256 * 4)));
}

SortRoute carve_route(const void* base, uint64_t n) {
  const uint64_t tiles = (n + kSortTile - 1) / kSortTile;
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

template <int W>
static hipError_t route_pass(bool fwd, const SortRoute& r, int k, uint64_t n, const float* in, float* out, hipStream_t s) {
  static const char* const kFwd[5] = {"", "k_route_fwd_w1", "k_route_fwd_w2", "k_route_fwd_w3", "k_route_fwd_w4"};
  static const char* const kInv[5] = {"", "k_route_inv_w1", "k_route_inv_w2", "k_route_inv_w3", "k_route_inv_w4"};
  const uint64_t tiles = (n + kSortTile - 1) / kSortTile;
  if (fwd)
    LAPLEX_LAUNCH(kFwd[W], n, s,
                  k_route_fwd<W><<<dim3((unsigned)tiles), dim3(kSortBlock), 0, s>>>(in, out, r.lpos[k], r.dstart[k], r.gbase[k], n));
  else
    LAPLEX_LAUNCH(kInv[W], n, s,
                  k_route_inv<W><<<dim3((unsigned)tiles), dim3(kSortBlock), 0, s>>>(in, out, r.lpos[k], r.dstart[k], r.gbase[k], n));
  return hipGetLastError();
}

static hipError_t route_pass_w(bool fwd, const SortRoute& r, int k, uint64_t n, uint32_t W, const float* in, float* out,
                               hipStream_t s) {
  switch (W) {
    case 1: return route_pass<1>(fwd, r, k, n, in, out, s);
    case 2: return route_pass<2>(fwd, r, k, n, in, out, s);
    case 3: return route_pass<3>(fwd, r, k, n, in, out, s);
    case 4: return route_pass<4>(fwd, r, k, n, in, out, s);
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

}  // namespace laplex
