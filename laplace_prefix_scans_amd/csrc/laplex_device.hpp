// Device helpers shared by the LAPLEX kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace laplex {

constexpr int kWave = 64;

// ---------------------------------------------------------------- float keys
// Order-preserving map from float bits to unsigned keys.  -0.0 is mapped to
// the key of +0.0 so that the two compare equal (a stable sort then keeps
// them in input order).
__device__ __forceinline__ uint32_t float_to_key(uint32_t u) {
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t key_to_float_bits(uint32_t k) {
  return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
}
constexpr uint32_t kKeyPlusZero = 0x80000000u;
__device__ __forceinline__ bool bits_nonfinite(uint32_t u) { return (u & 0x7F800000u) == 0x7F800000u; }

// ---------------------------------------------------------------- lanes
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }
// number of set bits of `mask` in lanes strictly below this lane
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Lanes of the wave whose 8-bit digit equals this lane's digit (within `valid`).
__device__ __forceinline__ uint64_t match_digit8(uint32_t d, uint64_t valid) {
  uint64_t peers = valid;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// ---------------------------------------------------------------- coherent status words
// Relaxed agent-scope atomics: the value read is the one in the device's
// coherent memory, visible across XCDs.
template <typename T>
__device__ __forceinline__ T load_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void store_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- exp
// e^x for x <= 0 as 2^(x log2 e) on the hardware exp2 unit.  The argument is
// always a difference of two anchors taken in float first, so every factor
// is <= 1 and never a product of decays.
__device__ __forceinline__ float decay(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Decay in one of two modes.  TIE: the zero-temperature limit of the kernel,
// exp(x / T) as T -> 0 for x <= 0, i.e. 1 between equal anchors and 0 otherwise;
// scanned with it, the recurrences sum within groups of tied anchors only.
template <bool TIE>
__device__ __forceinline__ float decay_m(float x) {
  if constexpr (TIE)
    return x == 0.f ? 1.f : 0.f;
  else
    return decay(x);
}
// the same with the mode chosen at run time (uniform per block)
__device__ __forceinline__ float decay_r(float x, bool tie) { return tie ? (x == 0.f ? 1.f : 0.f) : decay(x); }

// ---------------------------------------------------------------- affine segment scans
// A segment of the forward recurrence L_i = x_i + exp(s_{i-1} - s_i) L_{i-1}
// is summarised by (B, s): its last value with zero carry-in, and the anchor
// of its last element.  Joining (B_l, s_l) then (B_r, s_r) gives
// (B_r + exp(s_l - s_r) B_l, s_r).  The backward recurrence is the mirror
// image, summarised by the anchor of the segment's first element.

// Inclusive forward scan across the wave, lane order.  `s` is this lane's
// segment-end anchor (it does not change).
template <int C, bool TIE = false>
__device__ __forceinline__ void wave_scan_fwd(float (&B)[C], float s) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float sl = __shfl_up(s, off);
    const float w = decay_m<TIE>(sl - s);
    const bool take = lane >= off;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float bl = __shfl_up(B[c], off);
      if (take) B[c] = fmaf(w, bl, B[c]);
    }
  }
}

// Inclusive backward scan across the wave (from the last lane down).  `s` is
// this lane's segment-start anchor.
template <int C, bool TIE = false>
__device__ __forceinline__ void wave_scan_bwd(float (&B)[C], float s) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float sr = __shfl_down(s, off);
    const float w = decay_m<TIE>(s - sr);
    const bool take = lane + off < kWave;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float br = __shfl_down(B[c], off);
      if (take) B[c] = fmaf(w, br, B[c]);
    }
  }
}

// Deterministic wave sum (butterfly).
template <int C>
__device__ __forceinline__ void wave_sum(float (&v)[C]) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] += __shfl_xor(v[c], off);
  }
}

}  // namespace laplex
