// CPU emulation of the HIP execution model for running the library's device
// code on the host (test infrastructure; never part of liblaplex.so).
//
// Every GPU thread is one OS thread.  __syncthreads is a pthread barrier over
// the workgroup.  Every cross-lane operation (DPP row shifts, shuffles,
// readlane, ballot) is an exchange through a per-wave slot array between two
// crossings of a per-wave pthread barrier, so the 64 lanes of a wave see each
// other's values exactly as they would in lockstep, and ThreadSanitizer sees
// the happens-before edges of exactly those synchronisations: any other
// communication between threads through memory without a barrier is reported
// as a data race.  Workgroups of a launch run one after another.
//
// __shared__ arrays are function-local statics placed in one linker section,
// which the launcher fills with a poison pattern before every workgroup, so a
// read of shared memory that the workgroup has not written shows up in the
// output.
#pragma once
#include <pthread.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct float2 { float x, y; };
struct float4 { float x, y, z, w; };
struct uint2 { unsigned x, y; };
struct uint4 { unsigned x, y, z, w; };
inline float2 make_float2(float a, float b) { return {a, b}; }
inline float4 make_float4(float a, float b, float c, float d) { return {a, b, c, d}; }
inline uint2 make_uint2(unsigned a, unsigned b) { return {a, b}; }
inline uint4 make_uint4(unsigned a, unsigned b, unsigned c, unsigned d) { return {a, b, c, d}; }

typedef int hipError_t;
constexpr hipError_t hipSuccess = 0;
typedef struct simt_stream* hipStream_t;

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static __attribute__((section("simt_lds")))

extern "C" char __start_simt_lds[], __stop_simt_lds[];

namespace simt {
constexpr int kLanes = 64;

struct Wave {
  pthread_barrier_t bar;
  uint64_t slot[2][kLanes];
};
struct Block {
  pthread_barrier_t bar;
};
struct Ctx {
  dim3 tid, bid, bdim, gdim;
  int lane = 0;
  int parity = 0;
  Wave* wave = nullptr;
  Block* block = nullptr;
};
inline thread_local Ctx g_ctx;

// One exchange: publish v, wait for the wave, return the value lane `src`
// published.  Two slot buffers alternate, so one barrier per exchange
// suffices: the buffer written by exchange k + 2 is read by exchange k only
// before every lane has crossed the barrier of exchange k + 1.
inline void publish_wait(uint64_t v) {
  Ctx& c = g_ctx;
  c.wave->slot[c.parity][c.lane] = v;
  pthread_barrier_wait(&c.wave->bar);
}
inline uint64_t slot_of(int src) { return g_ctx.wave->slot[g_ctx.parity][src & (kLanes - 1)]; }
inline void done() { g_ctx.parity ^= 1; }

template <typename T>
inline uint64_t to_bits(T v) {
  static_assert(sizeof(T) <= 8, "exchange of at most 8 bytes");
  uint64_t b = 0;
  std::memcpy(&b, &v, sizeof(T));
  return b;
}
template <typename T>
inline T from_bits(uint64_t b) {
  T v;
  std::memcpy(&v, &b, sizeof(T));
  return v;
}
template <typename T>
inline T read_lane(T v, int src) {
  publish_wait(to_bits(v));
  const T r = from_bits<T>(slot_of(src));
  done();
  return r;
}
// DPP within 16-lane rows: row_shr:k (0x110 | k) and row_shl:k (0x100 | k),
// where a lane whose source lies outside its row gets 0 with the bound
// control (bc) and keeps `old` without it; row_ror:k (0x120 | k, lane i
// reads lane i - k mod 16 of its row); row_mirror (0x140); row_half_mirror
// (0x141, within each half-row); quad_perm (0x00-0xFF: lane i of a quad
// reads lane (ctrl >> 2i) & 3 of it).
inline int dpp(int old, int src, int ctrl, bool bc) {
  const int l = g_ctx.lane, rl = l & 15, row0 = l & ~15;
  int from = -1;
  if (ctrl >= 0 && ctrl <= 0xFF) {
    from = (l & ~3) | ((ctrl >> (2 * (l & 3))) & 3);
  } else if ((ctrl & 0xFF0) == 0x110) {
    const int k = ctrl & 15;
    if (rl >= k) from = l - k;
  } else if ((ctrl & 0xFF0) == 0x100) {
    const int k = ctrl & 15;
    if (rl + k <= 15) from = l + k;
  } else if ((ctrl & 0xFF0) == 0x120) {
    from = row0 | ((rl - (ctrl & 15)) & 15);
  } else if (ctrl == 0x140) {
    from = row0 | (15 - rl);
  } else if (ctrl == 0x141) {
    from = (l & ~7) | (7 - (l & 7));
  } else {
    std::fprintf(stderr, "simt: DPP control 0x%x not emulated\n", ctrl);
    std::abort();
  }
  publish_wait(to_bits(src));
  const int r = from >= 0 ? from_bits<int>(slot_of(from)) : (bc ? 0 : old);
  done();
  return r;
}
// The lane-swap instructions: permlane32_swap(a, b) gives {lanes 0-31 of a
// then lanes 0-31 of b, lanes 32-63 of a then lanes 32-63 of b};
// permlane16_swap(a, b) gives {rows 0, 2 of a interleaved with rows 0, 2 of
// b, rows 1, 3 of a interleaved with rows 1, 3 of b} (rows of 16 lanes).
struct u32x2 {
  unsigned v[2];
  unsigned operator[](int i) const { return v[i]; }
};
inline u32x2 permlane_swap(unsigned a, unsigned b, int half) {
  const int l = g_ctx.lane;
  const bool hi = (l & half) != 0;
  // r0: own a in the low part, b of the lane `half` below in the high part;
  // r1: a of the lane `half` above in the low part, own b in the high part
  const unsigned a_up = read_lane<unsigned>(a, hi ? l : l + half);
  const unsigned b_dn = read_lane<unsigned>(b, hi ? l - half : l);
  u32x2 r;
  r.v[0] = hi ? b_dn : a;
  r.v[1] = hi ? b : a_up;
  return r;
}
inline uint64_t ballot(bool p) {
  publish_wait(p ? 1u : 0u);
  uint64_t m = 0;
  for (int i = 0; i < kLanes; ++i) m |= (g_ctx.wave->slot[g_ctx.parity][i] & 1u) << i;
  done();
  return m;
}

// Fill the shared-memory section with a poison byte pattern.
inline unsigned& lds_poison() {
  static unsigned p = 0x7FC0DEADu;
  return p;
}
inline void poison_lds() {
  const unsigned p = lds_poison();
  for (char* q = __start_simt_lds; q + 4 <= __stop_simt_lds; q += 4) std::memcpy(q, &p, 4);
}

// Run `body` for every workgroup of grid (x, y) whose flat index `keep`
// accepts, one workgroup at a time: block.x threads are started once per
// launch and step through the workgroups together (a barrier before and
// after each, the shared memory poisoned in between).
template <typename F, typename K>
void launch(dim3 grid, dim3 block, F body, K keep) {
  const unsigned nt = block.x;
  if (nt % kLanes != 0) {
    std::fprintf(stderr, "simt: workgroup size %u is not a multiple of %d\n", nt, kLanes);
    std::abort();
  }
  std::vector<dim3> blocks;
  for (unsigned by = 0; by < grid.y; ++by)
    for (unsigned bx = 0; bx < grid.x; ++bx)
      if (keep((uint64_t)by * grid.x + bx)) blocks.push_back(dim3(bx, by));
  if (blocks.empty()) return;
  const unsigned nw = nt / kLanes;
  Block b;
  pthread_barrier_init(&b.bar, nullptr, nt);
  pthread_barrier_t step;
  pthread_barrier_init(&step, nullptr, nt);
  std::vector<Wave> waves(nw);
  for (auto& w : waves) pthread_barrier_init(&w.bar, nullptr, kLanes);
  std::vector<std::thread> ts;
  ts.reserve(nt);
  for (unsigned t = 0; t < nt; ++t)
    ts.emplace_back([&, t] {
      Ctx& c = g_ctx;
      c.tid = dim3(t);
      c.bdim = block;
      c.gdim = grid;
      c.lane = (int)(t % kLanes);
      c.wave = &waves[t / kLanes];
      c.block = &b;
      for (const dim3& bid : blocks) {
        if (t == 0) poison_lds();
        pthread_barrier_wait(&step);
        c.bid = bid;
        c.parity = 0;
        body();
        pthread_barrier_wait(&step);
      }
    });
  for (auto& th : ts) th.join();
  for (auto& w : waves) pthread_barrier_destroy(&w.bar);
  pthread_barrier_destroy(&step);
  pthread_barrier_destroy(&b.bar);
}
template <typename F>
void launch(dim3 grid, dim3 block, F body) {
  launch(grid, block, body, [](uint64_t) { return true; });
}
}  // namespace simt

#define threadIdx (::simt::g_ctx.tid)
#define blockIdx (::simt::g_ctx.bid)
#define blockDim (::simt::g_ctx.bdim)
#define gridDim (::simt::g_ctx.gdim)
#define __syncthreads() pthread_barrier_wait(&::simt::g_ctx.block->bar)
#define __lane_id() (::simt::g_ctx.lane)
#define __builtin_amdgcn_exp2f(x) exp2f(x)
#define __builtin_amdgcn_update_dpp(old, src, ctrl, rm, bm, bc) ::simt::dpp((old), (src), (ctrl), (bc))
#define __builtin_amdgcn_permlane32_swap(a, b, fi, bc) ::simt::permlane_swap((a), (b), 32)
#define __builtin_amdgcn_permlane16_swap(a, b, fi, bc) ::simt::permlane_swap((a), (b), 16)
#define __builtin_amdgcn_readfirstlane(x) ::simt::read_lane<int>((x), 0)
#define __builtin_amdgcn_readlane(x, l) ::simt::read_lane<int>((x), (l))

namespace simt {
inline uint32_t mbcnt_lo(uint32_t mask, uint32_t acc) {
  const int l = std::min(g_ctx.lane, 32);
  const uint32_t below = l >= 32 ? 0xFFFFFFFFu : ((1u << l) - 1u);
  return acc + (uint32_t)__builtin_popcount(mask & below);
}
inline uint32_t mbcnt_hi(uint32_t mask, uint32_t acc) {
  const int l = std::max(g_ctx.lane - 32, 0);
  const uint32_t below = l >= 32 ? 0xFFFFFFFFu : ((1u << l) - 1u);
  return acc + (uint32_t)__builtin_popcount(mask & below);
}
}  // namespace simt
#define __builtin_amdgcn_mbcnt_lo(m, a) ::simt::mbcnt_lo((m), (a))
#define __builtin_amdgcn_mbcnt_hi(m, a) ::simt::mbcnt_hi((m), (a))
inline uint64_t __ballot(int p) { return ::simt::ballot(p != 0); }

// HIP's shuffles at width 64: a lane whose source is out of range reads itself.
template <typename T>
inline T __shfl(T v, int src) {
  return ::simt::read_lane<T>(v, src & 63);
}
template <typename T>
inline T __shfl_up(T v, unsigned d) {
  const int l = ::simt::g_ctx.lane;
  return ::simt::read_lane<T>(v, (l >= (int)d) ? l - (int)d : l);
}
template <typename T>
inline T __shfl_down(T v, unsigned d) {
  const int l = ::simt::g_ctx.lane;
  return ::simt::read_lane<T>(v, (l + (int)d < 64) ? l + (int)d : l);
}
template <typename T>
inline T __shfl_xor(T v, int mask) {
  const int l = ::simt::g_ctx.lane;
  const int s = l ^ mask;
  return ::simt::read_lane<T>(v, s < 64 ? s : l);
}

#define __HIP_MEMORY_SCOPE_AGENT 0
#define __hip_atomic_load(p, order, scope) __atomic_load_n((p), (order))
#define __hip_atomic_store(p, v, order, scope) __atomic_store_n((p), (v), (order))
