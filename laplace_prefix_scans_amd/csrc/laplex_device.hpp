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

// ---------------------------------------------------------------- tile placement
// Tile of this block.  Workgroups are dispatched to the 8 XCDs round-robin, so
// block b runs on XCD b % 8; giving each XCD a contiguous range of tiles puts
// neighbouring tiles -- whose digit runs share cache lines at their ends --
// behind the same L2.  Launch ceil(tiles / 8) * 8 blocks; returns false for
// the few padding blocks.
constexpr unsigned kXcds = 8;
__device__ __forceinline__ bool xcd_tile(uint64_t tiles, uint64_t& tile) {
  const uint64_t per = (tiles + kXcds - 1) / kXcds;
  tile = (uint64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  return tile < tiles;
}
inline uint64_t xcd_blocks(uint64_t tiles) { return ((tiles + kXcds - 1) / kXcds) * kXcds; }

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

// Value of a lane in the same 16-lane row, by DPP: CTRL 0x110 | k reads lane
// - k (row_shr), 0x100 | k reads lane + k (row_shl).  A lane whose source lies
// outside its row reads 0 (the callers mask it): the bound control makes the
// hardware supply the 0, so no register has to be cleared first.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Inclusive prefix sum of u32 values over the wave: DPP row shifts within
// each 16-lane row, then the row totals joined (lane 15 of each row, and of
// the lower half, read by shuffles).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_incl_sum_u32(uint32_t x) {
  const int lane = lane_id(), rl = lane & 15, row = lane >> 4;
  uint32_t t;
  t = dpp_row_u32<0x110 | 1>(x);
  x += rl >= 1 ? t : 0u;
  t = dpp_row_u32<0x110 | 2>(x);
  x += rl >= 2 ? t : 0u;
  t = dpp_row_u32<0x110 | 4>(x);
  x += rl >= 4 ? t : 0u;
  t = dpp_row_u32<0x110 | 8>(x);
  x += rl >= 8 ? t : 0u;
  t = (uint32_t)__shfl(x, (lane & ~31) + 15);
  x += (row & 1) ? t : 0u;
  t = (uint32_t)__shfl(x, 31);
  x += row >= 2 ? t : 0u;
  return x;
}

// One scan step: the lanes with `take` join the segment summary (bs, ss) that
// precedes (forward) or follows (backward) them.
// Columns [0, NT) of a scan use the tie decay, columns [NT, C) the kernel's
// decay (NT = C: all tie; NT = 0: all kernel); both weights come from the
// same anchor difference.
template <int C, int NT, bool FWD>
__device__ __forceinline__ void scan_join(float (&B)[C], float s, const float (&bs)[C], float ss, bool take) {
  const float x = FWD ? ss - s : s - ss;
  const float wt = NT > 0 ? decay_m<true>(x) : 0.f;
  const float we = NT < C ? decay_m<false>(x) : 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (take) B[c] = fmaf(c < NT ? wt : we, bs[c], B[c]);
}

// The same join for a DPP row step, whose lanes that do not take it read 0
// (their source lies outside the row): masking the two weights then leaves
// those lanes' values as they are (0 * 0 is added), without a select per
// column.
template <int C, int NT, bool FWD>
__device__ __forceinline__ void scan_join_row(float (&B)[C], float s, const float (&bs)[C], float ss, bool take) {
  const float x = FWD ? ss - s : s - ss;
  const float wt = NT > 0 && take ? decay_m<true>(x) : 0.f;
  const float we = NT < C && take ? decay_m<false>(x) : 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) B[c] = fmaf(c < NT ? wt : we, bs[c], B[c]);
}

// Inclusive forward scan across the wave, lane order.  `s` is this lane's
// segment-end anchor (it does not change).  Within each 16-lane row a
// Hillis-Steele scan by DPP row shifts; then rows 1 and 3 join the total of
// the row before (lanes 15 and 47), and rows 2 and 3 the total of rows 0-1
// (lane 31).  NT: leading columns with the tie decay.
template <int C, int NT>
__device__ __forceinline__ void wave_scan_fwd_mix(float (&B)[C], float s) {
  const int lane = lane_id(), rl = lane & 15, row = lane >> 4;
  float bs[C];
#define LAPLEX_FWD_STEP(K)                                              \
  {                                                                     \
    const float ss = dpp_row<0x110 | K>(s);                             \
    _Pragma("unroll") for (int c = 0; c < C; ++c) bs[c] = dpp_row<0x110 | K>(B[c]); \
    scan_join_row<C, NT, true>(B, s, bs, ss, rl >= K);                  \
  }
  LAPLEX_FWD_STEP(1)
  LAPLEX_FWD_STEP(2)
  LAPLEX_FWD_STEP(4)
  LAPLEX_FWD_STEP(8)
#undef LAPLEX_FWD_STEP
  {
    const int src = (lane & ~31) + 15;  // row 1 reads lane 15, row 3 lane 47
    const float ss = __shfl(s, src);
#pragma unroll
    for (int c = 0; c < C; ++c) bs[c] = __shfl(B[c], src);
    scan_join<C, NT, true>(B, s, bs, ss, (row & 1) != 0);
  }
  {
    const float ss = __shfl(s, 31);
#pragma unroll
    for (int c = 0; c < C; ++c) bs[c] = __shfl(B[c], 31);
    scan_join<C, NT, true>(B, s, bs, ss, row >= 2);
  }
}
template <int C, bool TIE = false>
__device__ __forceinline__ void wave_scan_fwd(float (&B)[C], float s) {
  wave_scan_fwd_mix<C, TIE ? C : 0>(B, s);
}

// Inclusive backward scan across the wave (from the last lane down).  `s` is
// this lane's segment-start anchor.  The mirror image of the forward scan:
// row_shl steps within rows, then rows 0 and 2 join the row after (lanes 16
// and 48), and rows 0 and 1 the total of rows 2-3 (lane 32).
template <int C, int NT>
__device__ __forceinline__ void wave_scan_bwd_mix(float (&B)[C], float s) {
  const int lane = lane_id(), rl = lane & 15, row = lane >> 4;
  float bs[C];
#define LAPLEX_BWD_STEP(K)                                              \
  {                                                                     \
    const float ss = dpp_row<0x100 | K>(s);                             \
    _Pragma("unroll") for (int c = 0; c < C; ++c) bs[c] = dpp_row<0x100 | K>(B[c]); \
    scan_join_row<C, NT, false>(B, s, bs, ss, rl + K < 16);             \
  }
  LAPLEX_BWD_STEP(1)
  LAPLEX_BWD_STEP(2)
  LAPLEX_BWD_STEP(4)
  LAPLEX_BWD_STEP(8)
#undef LAPLEX_BWD_STEP
  {
    const int src = (lane & ~31) + 16;  // row 0 reads lane 16, row 2 lane 48
    const float ss = __shfl(s, src);
#pragma unroll
    for (int c = 0; c < C; ++c) bs[c] = __shfl(B[c], src);
    scan_join<C, NT, false>(B, s, bs, ss, (row & 1) == 0);
  }
  {
    const float ss = __shfl(s, 32);
#pragma unroll
    for (int c = 0; c < C; ++c) bs[c] = __shfl(B[c], 32);
    scan_join<C, NT, false>(B, s, bs, ss, row < 2);
  }
}
template <int C, bool TIE = false>
__device__ __forceinline__ void wave_scan_bwd(float (&B)[C], float s) {
  wave_scan_bwd_mix<C, TIE ? C : 0>(B, s);
}

// Deterministic wave sum: row prefix sums by DPP row shifts (lane 15 of each
// 16-lane row then holds its row's total), and the four row totals read as
// uniform values and added in a fixed order, so every lane gets the same bits.
template <int C>
__device__ __forceinline__ void wave_sum(float (&v)[C]) {
  const int rl = lane_id() & 15;
#define LAPLEX_SUM_STEP(K)                                   \
  _Pragma("unroll") for (int c = 0; c < C; ++c) {            \
    const float t = dpp_row<0x110 | K>(v[c]);                \
    if (rl >= K) v[c] += t;                                  \
  }
  LAPLEX_SUM_STEP(1)
  LAPLEX_SUM_STEP(2)
  LAPLEX_SUM_STEP(4)
  LAPLEX_SUM_STEP(8)
#undef LAPLEX_SUM_STEP
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int b = __builtin_bit_cast(int, v[c]);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 15));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 31));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 47));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 63));
    v[c] = (r0 + r1) + (r2 + r3);
  }
}

// Sums over the wave of N values that every lane holds (N a power of two, at
// most 32), transposed: at each of six levels a lane is paired with a
// partner (32 lanes apart, then 16, by the lane-swap instructions; then 8
// apart, within half-rows, within quads and in pairs, by DPP row
// permutations).  While a lane holds more than one value, it keeps half of
// them and adds the partner's copies of those, and the partner keeps the
// other half; once one value is left, a level adds the partner's copy.  The
// lane then holds the wave's sum of value (lane >> (6 - log2 N)); lanes that
// hold the same value hold the same bits (a + b and b + a are equal), and
// the order of the additions is fixed.  About 2N + 6 instructions, where
// summing each value by its own row scan and lane reads takes 11 each.
template <int CTRL, int NIN, int NOUT, int N>
__device__ __forceinline__ void wave_sum_t_level(float (&v)[N], bool hi) {
#pragma unroll
  for (int j = 0; j < NOUT; ++j) {
    if constexpr (NIN > 1) {
      const float keep = hi ? v[j + NOUT] : v[j], send = hi ? v[j] : v[j + NOUT];
      v[j] = keep + dpp_row<CTRL>(send);
    } else {
      v[j] = v[j] + dpp_row<CTRL>(v[j]);
    }
  }
}
template <int N>
__device__ __forceinline__ float wave_sum_t(float (&v)[N]) {
  static_assert(N >= 1 && N <= 32 && (N & (N - 1)) == 0, "a power of two, at most 32");
  constexpr int N1 = N > 1 ? N / 2 : 1, N2 = N1 > 1 ? N1 / 2 : 1, N3 = N2 > 1 ? N2 / 2 : 1, N4 = N3 > 1 ? N3 / 2 : 1,
                N5 = N4 > 1 ? N4 / 2 : 1;
  const int lane = lane_id();
  auto bits = [](float x) { return __builtin_bit_cast(unsigned, x); };
  auto flt = [](unsigned x) { return __builtin_bit_cast(float, x); };
  // 32 apart: the first result holds lanes 0-31 of the first operand and
  // lanes 0-31 of the second; the other result their lanes 32-63
#pragma unroll
  for (int j = 0; j < N1; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(bits(v[j]), bits(v[N > 1 ? j + N1 : j]), false, false);
    v[j] = flt(r[0]) + flt(r[1]);
  }
  // 16 apart: rows (16 lanes) 0 and 2 of the first result come from the
  // first operand, rows 1 and 3 from the second; the other result likewise
  // from the odd rows
#pragma unroll
  for (int j = 0; j < N2; ++j) {
    const auto r = __builtin_amdgcn_permlane16_swap(bits(v[j]), bits(v[N1 > 1 ? j + N2 : j]), false, false);
    v[j] = flt(r[0]) + flt(r[1]);
  }
  wave_sum_t_level<0x128, N2, N3>(v, (lane & 8) != 0);  // row rotated by 8: lanes 8 apart
  wave_sum_t_level<0x141, N3, N4>(v, (lane & 4) != 0);  // half-row mirror: l and 7 - l
  wave_sum_t_level<0x1B, N4, N5>(v, (lane & 2) != 0);   // quad [3,2,1,0]
  wave_sum_t_level<0xB1, N5, 1>(v, (lane & 1) != 0);    // quad [1,0,3,2]
  return v[0];
}

}  // namespace laplex
