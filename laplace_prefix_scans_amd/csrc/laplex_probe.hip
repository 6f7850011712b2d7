// Memory-system probes (liblaplex_probe.so): the streaming patterns the
// operator's kernels are measured against.  Not part of the operator.
#include "../../include/laplex_probe.h"

#include "laplex_device.hpp"

namespace laplex {
namespace {

constexpr int kProbeBlock = 256;   // threads of the one-piece shapes (4 KiB per workgroup)
constexpr int kCopy8Pieces = 8;    // 16-byte pieces per thread of COPY_8
constexpr int kRunTile = 8192;     // 8-byte pairs per tile of RUNS
constexpr int kRunBlock = 512;
constexpr int kRunLen = kRunTile / 256;

__global__ __launch_bounds__(kProbeBlock) void k_probe_copy1(const float4* __restrict__ in, float4* __restrict__ out,
                                                            uint64_t pieces) {
  uint64_t c;
  if (!xcd_tile((pieces + kProbeBlock - 1) / kProbeBlock, c)) return;
  const uint64_t i = c * kProbeBlock + threadIdx.x;
  if (i < pieces) out[i] = in[i];
}

__global__ __launch_bounds__(kProbeBlock) void k_probe_copy8(const float4* __restrict__ in, float4* __restrict__ out,
                                                            uint64_t pieces) {
  const uint64_t base = (uint64_t)blockIdx.x * kProbeBlock * kCopy8Pieces + threadIdx.x;
  float4 v[kCopy8Pieces];
#pragma unroll
  for (int u = 0; u < kCopy8Pieces; ++u) {
    const uint64_t i = base + (uint64_t)u * kProbeBlock;
    v[u] = i < pieces ? in[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int u = 0; u < kCopy8Pieces; ++u) {
    const uint64_t i = base + (uint64_t)u * kProbeBlock;
    if (i < pieces) out[i] = v[u];
  }
}

__global__ __launch_bounds__(kProbeBlock) void k_probe_read(const float4* __restrict__ in, float* __restrict__ sums,
                                                           uint64_t pieces) {
  __shared__ float s_part[kProbeBlock / kWave];
  uint64_t c;
  if (!xcd_tile((pieces + kProbeBlock - 1) / kProbeBlock, c)) return;
  const uint64_t i = c * kProbeBlock + threadIdx.x;
  const float4 v = i < pieces ? in[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  float s = (v.x + v.y) + (v.z + v.w);
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane_id() == 0) s_part[threadIdx.x / kWave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kProbeBlock / kWave; ++w) t += s_part[w];
    sums[c] = t;
  }
}

__global__ __launch_bounds__(kProbeBlock) void k_probe_write(float4* __restrict__ out, uint64_t pieces) {
  uint64_t c;
  if (!xcd_tile((pieces + kProbeBlock - 1) / kProbeBlock, c)) return;
  const uint64_t i = c * kProbeBlock + threadIdx.x;
  if (i < pieces) out[i] = make_float4(1.f, 2.f, 3.f, 4.f);
}

__global__ __launch_bounds__(kRunBlock) void k_probe_runs(const uint2* __restrict__ in, uint2* __restrict__ out,
                                                         uint64_t tiles) {
  constexpr int E = kRunTile / kRunBlock;
  const uint64_t t = blockIdx.x;
  uint2 v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = in[t * kRunTile + (uint64_t)e * kRunBlock + threadIdx.x];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t i = (uint32_t)(e * kRunBlock + threadIdx.x);  // tile-local pair
    const uint32_t d = i / kRunLen, j = i % kRunLen;
    out[((uint64_t)d * tiles + t) * kRunLen + j] = v[e];
  }
}

}  // namespace
}  // namespace laplex

extern "C" int laplex_probe(int kind, const void* src, void* dst, size_t bytes, hipStream_t stream) {
  using namespace laplex;
  if (dst == nullptr || (kind != LAPLEX_PROBE_WRITE && src == nullptr)) return 1;
  if ((reinterpret_cast<uintptr_t>(dst) & 15) || (src && (reinterpret_cast<uintptr_t>(src) & 15))) return 3;
  if (kind < LAPLEX_PROBE_COPY_1 || kind > LAPLEX_PROBE_RUNS) return 9;
  if (bytes % 16 || (kind == LAPLEX_PROBE_RUNS && bytes % ((size_t)kRunTile * 8))) return 2;
  if (bytes == 0) return 0;
  const uint64_t pieces = bytes / 16;
  const uint64_t chunks = (pieces + kProbeBlock - 1) / kProbeBlock;
  const float4* in = static_cast<const float4*>(src);
  float4* out = static_cast<float4*>(dst);
  switch (kind) {
    case LAPLEX_PROBE_COPY_1:
      k_probe_copy1<<<dim3((unsigned)xcd_blocks(chunks)), dim3(kProbeBlock), 0, stream>>>(in, out, pieces);
      break;
    case LAPLEX_PROBE_COPY_8: {
      const uint64_t per = (uint64_t)kProbeBlock * kCopy8Pieces;
      k_probe_copy8<<<dim3((unsigned)((pieces + per - 1) / per)), dim3(kProbeBlock), 0, stream>>>(in, out, pieces);
      break;
    }
    case LAPLEX_PROBE_READ:
      k_probe_read<<<dim3((unsigned)xcd_blocks(chunks)), dim3(kProbeBlock), 0, stream>>>(in, static_cast<float*>(dst), pieces);
      break;
    case LAPLEX_PROBE_WRITE:
      k_probe_write<<<dim3((unsigned)xcd_blocks(chunks)), dim3(kProbeBlock), 0, stream>>>(out, pieces);
      break;
    default: {
      const uint64_t tiles = bytes / ((size_t)kRunTile * 8);
      k_probe_runs<<<dim3((unsigned)tiles), dim3(kRunBlock), 0, stream>>>(static_cast<const uint2*>(src),
                                                                         static_cast<uint2*>(dst), tiles);
      break;
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
