// Stable LSD radix sort of float anchors with their permutation ("after
// sorting the anchors": LAPLEX technical summary, section 2.2, symmetric case).
//
// Keys are the order-preserving unsigned image of the float bits (-0.0 made
// equal to +0.0).  One read of the anchors builds all four 8-bit digit
// histograms and, for the first pass, each tile's digit counts; then four
// single-pass ("onesweep") scatter passes, each tile ranking its keys stably
// in LDS.  The first pass takes its tiles' global offsets from a scan of the
// per-tile counts; the later passes, whose tiles' contents are only known once
// the previous pass has run, publish per-digit counts and look back over
// earlier tiles (decoupled look-back).  Pass 1 generates the identity
// permutation itself; pass 4 writes the sorted anchors and the permutation.
#include <cstdlib>

#include "laplex_kernels.hpp"

namespace laplex {

// ------------------------------------------------------------------ status words
template <typename ST>
struct Status;
template <>
struct Status<uint32_t> {  // n <= 2^30: 2-bit flag, 30-bit count
  static __device__ __forceinline__ uint32_t pack(uint32_t flag, uint32_t v) { return (flag << 30) | (v & 0x3FFFFFFFu); }
  static __device__ __forceinline__ uint32_t flag(uint32_t w) { return w >> 30; }
  static __device__ __forceinline__ uint32_t value(uint32_t w) { return w & 0x3FFFFFFFu; }
};
template <>
struct Status<uint64_t> {  // n < 2^32: flag in the high word, count in the low word
  static __device__ __forceinline__ uint64_t pack(uint32_t flag, uint32_t v) { return ((uint64_t)flag << 32) | v; }
  static __device__ __forceinline__ uint32_t flag(uint64_t w) { return (uint32_t)(w >> 32); }
  static __device__ __forceinline__ uint32_t value(uint64_t w) { return (uint32_t)w; }
};
constexpr uint32_t kFlagAggregate = 1, kFlagInclusive = 2;
constexpr uint32_t kSpinLimit = 1u << 22;

__global__ void k_fill_u32(uint32_t* __restrict__ p, uint64_t count, uint32_t value) {
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < count; i += stride) p[i] = value;
}

// ------------------------------------------------------------------ histograms
// All four digit histograms in one read.  Sub-histograms are replicated
// kHistRep times in LDS (lane % kHistRep picks one) so that keys sharing a
// digit (e.g. the top byte of anchors in a narrow range) do not all hit one
// LDS word.  Integer atomics: the result does not depend on ordering.
// One replica of every histogram per lane position (lane mod 32), so the 32
// lanes an LDS cycle serves always hit 32 different banks; 1024 threads keep
// enough loads in flight with one block per CU.
// The same read also counts the first pass's digit in each 8192-key sort tile
// (sorts with smaller tiles look back in every pass and ignore it): block
// b reads a contiguous range of chunks (two tiles each), keeps a running
// count per digit, and writes each tile's count of the tiles before it in
// the block's range (tcount) and the range's total (bsum[b]); an exclusive
// scan of bsum over blocks then completes the first pass's offsets, so that
// pass needs no look-back.  Tile counts are double-buffered by chunk parity
// (one barrier per chunk) and the next chunk's keys are loaded before it.
// The low digit's global histogram is the sum of the blocks' totals, so the
// per-key LDS atomics are the same four as for the four histograms alone.
constexpr int kHistRep = 32;
constexpr int kHistBlock = 1024;
constexpr int kHistItems = 16;
constexpr int kTileRep = 8;
static_assert(kHistBlock * kHistItems == 2 * kSortTile, "a histogram chunk is two sort tiles");

__global__ __launch_bounds__(kHistBlock) void k_sort_hist(const uint32_t* __restrict__ a_bits, uint64_t n,
                                                          uint32_t* __restrict__ hist, uint32_t* __restrict__ header,
                                                          uint32_t* __restrict__ tcount, uint32_t* __restrict__ bsum,
                                                          uint64_t chunks_per_block) {
  __shared__ uint32_t sh[3][256][kHistRep];     // digits 2..4
  __shared__ uint32_t st[2][2][256][kTileRep];  // digit 1: [chunk parity][tile of the chunk][digit][replica]
  for (int i = threadIdx.x; i < 3 * 256 * kHistRep; i += kHistBlock) (&sh[0][0][0])[i] = 0;
  for (int i = threadIdx.x; i < 2 * 2 * 256 * kTileRep; i += kHistBlock) (&st[0][0][0][0])[i] = 0;
  __syncthreads();
  const int rep = lane_id() % kHistRep, trep = lane_id() % kTileRep;
  const uint64_t tiles = (n + kSortTile - 1) / kSortTile;
  uint32_t bad = 0, run = 0;  // run: thread d < 256's count of digit d so far in this block's range
  const uint64_t chunk = (uint64_t)kHistBlock * kHistItems;
  const uint64_t nchunks = (n + chunk - 1) / chunk;
  const uint64_t c0 = (uint64_t)blockIdx.x * chunks_per_block;
  const uint64_t c1 = c0 + chunks_per_block < nchunks ? c0 + chunks_per_block : nchunks;
  // the next chunk's keys are loaded (clamped into range, so every load is
  // issued unconditionally) before this chunk's keys are counted; full
  // chunks are counted without per-key conditions, so that the compiler
  // waits only for this chunk's loads
  uint32_t nxt[kHistItems];
#pragma unroll
  for (int it = 0; it < kHistItems; ++it) {
    const uint64_t i = c0 * chunk + (uint64_t)it * kHistBlock + threadIdx.x;
    nxt[it] = a_bits[i < n ? i : n - 1];
  }
  for (uint64_t c = c0; c < c1; ++c) {
    const uint64_t base = c * chunk;
    const int par = (int)(c & 1);
    uint32_t u[kHistItems];
#pragma unroll
    for (int it = 0; it < kHistItems; ++it) u[it] = nxt[it];
#pragma unroll
    for (int it = 0; it < kHistItems; ++it) {
      const uint64_t i = base + chunk + (uint64_t)it * kHistBlock + threadIdx.x;
      nxt[it] = a_bits[i < n ? i : n - 1];
    }
    auto count = [&](int it, uint32_t bits) {
      bad |= bits_nonfinite(bits) ? 1u : 0u;
      const uint32_t k = float_to_key(bits);
      atomicAdd(&sh[0][(k >> 8) & 255u][rep], 1u);
      atomicAdd(&sh[1][(k >> 16) & 255u][rep], 1u);
      atomicAdd(&sh[2][k >> 24][rep], 1u);
      atomicAdd(&st[par][it / (kHistItems / 2)][k & 255u][trep], 1u);
    };
    if (base + chunk <= n) {
#pragma unroll
      for (int it = 0; it < kHistItems; ++it) count(it, u[it]);
    } else {
#pragma unroll
      for (int it = 0; it < kHistItems; ++it)
        if (base + (uint64_t)it * kHistBlock + threadIdx.x < n) count(it, u[it]);
    }
    __syncthreads();
    // (the buffer of this parity is next written two chunks on, after the
    // next iteration's barrier, which every thread reaches after this)
    if (threadIdx.x < 256) {
      const int d = threadIdx.x;
      uint32_t s0 = 0, s1 = 0;
#pragma unroll
      for (int r = 0; r < kTileRep; ++r) {
        s0 += st[par][0][d][(r + d) % kTileRep];
        s1 += st[par][1][d][(r + d) % kTileRep];
      }
#pragma unroll
      for (int r = 0; r < kTileRep; ++r) st[par][0][d][r] = st[par][1][d][r] = 0;
      const uint64_t t = 2 * c;
      if (t < tiles) tcount[t * 256 + d] = run;
      if (t + 1 < tiles) tcount[(t + 1) * 256 + d] = run + s0;
      run += s0 + s1;
    }
  }
  if (threadIdx.x < 256) {
    bsum[(uint64_t)blockIdx.x * 256 + threadIdx.x] = run;
    if (run) atomicAdd(&hist[threadIdx.x], run);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 3 * 256; i += kHistBlock) {
    uint32_t s = 0;
#pragma unroll
    for (int r = 0; r < kHistRep; ++r) s += sh[i >> 8][i & 255][(r + i) % kHistRep];
    if (s) atomicAdd(&hist[256 + i], s);
  }
  if (__ballot(bad) != 0ull && lane_id() == 0) atomicOr(&header[kHdrFlags], kFlagNonFinite);
}


// ------------------------------------------------------------------ offsets
// One 1024-thread block, after the histogram read:
//  * exclusive digit offsets of every pass (threads 0..255, thread d owning
//    digit value d), and per pass whether its tiles publish their digit
//    counts before ranking: only when no digit value holds more than 1/16 of
//    the keys, since the early count takes LDS atomic adds that serialise
//    when many lanes share a digit (the ranking itself does not);
//  * with `rows` > 0, the first pass's table: bsum[b][d] (digit d's count in
//    histogram block b's range) becomes its exclusive prefix over blocks,
//    thread (q, d) scanning digit d over the q-th quarter of the rows.
constexpr int kScanThreads = 1024;
constexpr int kScanQuarters = kScanThreads / 256;
constexpr uint64_t kTableMinTiles = 64;

__global__ __launch_bounds__(kScanThreads) void k_sort_offsets(const uint32_t* __restrict__ hist, uint32_t* __restrict__ offs,
                                                               uint32_t* __restrict__ header, uint32_t* __restrict__ bsum,
                                                               uint64_t rows) {
  __shared__ uint32_t wsum[4], wmax[4];
  __shared__ uint32_t part[kScanQuarters][256];
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int q = tid >> 8, d = tid & 255;
  for (int p = 0; p < 4; ++p) {
    uint32_t v = 0, x = 0;
    if (tid < 256) {
      v = hist[p * 256 + d];
      x = v;
      uint32_t mx = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_up(x, off);
        if (lane >= off) x += t;
        mx = max(mx, (uint32_t)__shfl_xor(mx, off));
      }
      if (lane == kWave - 1) wsum[w] = x;
      if (lane == 0) wmax[w] = mx;
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t pre = 0, total = 0, top = 0;
      for (int i = 0; i < 4; ++i) {
        if (i < w) pre += wsum[i];
        total += wsum[i];
        top = max(top, wmax[i]);
      }
      offs[p * 256 + d] = pre + x - v;
      if (d == 0) header[kHdrEarly0 + p] = (top <= total / 16) ? 1u : 0u;
    }
    __syncthreads();
  }
  if (rows == 0) return;
  const uint64_t seg = (rows + kScanQuarters - 1) / kScanQuarters;
  const uint64_t g0 = (uint64_t)q * seg < rows ? (uint64_t)q * seg : rows;
  const uint64_t g1 = g0 + seg < rows ? g0 + seg : rows;
  constexpr int B = 16;
  uint32_t sum = 0;
  for (uint64_t g = g0; g < g1; g += B) {
    uint32_t vv[B];
#pragma unroll
    for (int j = 0; j < B; ++j) vv[j] = (g + j < g1) ? bsum[(g + j) * 256 + d] : 0u;
#pragma unroll
    for (int j = 0; j < B; ++j) sum += vv[j];
  }
  part[q][d] = sum;
  __syncthreads();
  uint32_t run = 0;
  for (int i = 0; i < q; ++i) run += part[i][d];
  for (uint64_t g = g0; g < g1; g += B) {
    uint32_t vv[B];
#pragma unroll
    for (int j = 0; j < B; ++j) vv[j] = (g + j < g1) ? bsum[(g + j) * 256 + d] : 0u;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (g + j < g1) bsum[(g + j) * 256 + d] = run;
      run += vv[j];
    }
  }
}

// ------------------------------------------------------------------ onesweep pass
// MODE 0: input is the anchors' float bits (keys computed here, values are the
//         input indices); MODE 1: (key, value) pairs to pairs;
// MODE 2: pairs in; writes float bits of the sorted anchors and the permutation.
// PAY (MODE 0 and 2): the values are a payload of one 32-bit word per anchor
// (read from `pay` in input order) instead of the input indices, so pass 4
// writes the payload in sorted order where the permutation would go, and the
// sorted anchors carry +0.0 for -0.0 (no index to look the sign up by).
// Keys and values travel as interleaved pairs so that each digit run is one
// contiguous stretch of 8-byte elements.
// Threads 0..255 also own one digit value each for the per-digit steps (all
// of a 256-thread block, the first four waves of a 512-thread one).
constexpr int kLookback = 4;  // predecessor status words read per round trip (more costs more status traffic than it saves)

template <int MODE, typename ST, bool PAY, int TILE>
__global__ __launch_bounds__(sort_block(MODE, TILE)) __attribute__((amdgpu_waves_per_eu(MODE == 0 && TILE == kSortTile ? 6 : 4))) void k_onesweep(const uint2* __restrict__ kvin, uint2* __restrict__ kvout,
                                                         uint32_t* __restrict__ kout, uint32_t* __restrict__ vout,
                                                         const uint32_t* __restrict__ a_bits, ST* __restrict__ status,
                                                         uint32_t* __restrict__ header, int pass,
                                                         const uint32_t* __restrict__ digit_start, uint64_t n,
                                                         uint16_t* __restrict__ r_lpos, uint16_t* __restrict__ r_dstart,
                                                         uint32_t* __restrict__ r_gbase, const uint32_t* __restrict__ pay,
                                                         const uint32_t* __restrict__ tcount, const uint32_t* __restrict__ bpre,
                                                         uint64_t chunks_per_block, uint32_t spin_limit, bool publish) {
  static_assert(!PAY || MODE != 1, "the payload enters in pass 1 and leaves in pass 4");
  constexpr bool HOLDV = MODE != 0 || PAY;  // values held in registers (else recomputed input indices)
  constexpr int BLOCK = sort_block(MODE, TILE);
  static_assert(BLOCK % 256 == 0, "at least one thread per digit value");
  static_assert(TILE == kSortTile || TILE == kSortTileSmall, "a sort tile size");
  constexpr int E = TILE / BLOCK;
  constexpr int NW = BLOCK / kWave;
  // staging for half a tile, large enough for the ranking scratch too
  constexpr int kStage = TILE / 2 > NW * 256 * 2 ? TILE / 2 : NW * 256 * 2;
  __shared__ __align__(16) uint2 s_kv[kStage];
  __shared__ uint32_t s_whist[NW][256];
  __shared__ uint32_t s_gbase[256];
  __shared__ uint32_t s_wsum[4];
  __shared__ uint32_t s_tile;
  __shared__ uint32_t s_stop;
  __shared__ uint32_t s_thist[256];

  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  const uint32_t shift = 8u * (uint32_t)pass;
  // Ranking scratch, on top of s_kv (unused until the scatter): per wave and
  // digit value, {mask of the lanes holding that digit in the current
  // iteration (64 bits), the wave's running count of that digit, unused}.
  static_assert(NW * 256 * sizeof(uint4) <= sizeof(s_kv), "ranking scratch fits in the staging buffer");
  uint4* s_match = reinterpret_cast<uint4*>(s_kv);
  // With tcount (large first passes) the offsets come from the table made
  // by the histogram read, so tiles depend on no other tile and are placed
  // by block index; otherwise tiles are taken in ticket order for the
  // look-back.
  const bool table = MODE == 0 && TILE == kSortTile && tcount != nullptr;
  uint64_t xtile = 0;
  if (table && !xcd_tile((n + TILE - 1) / TILE, xtile)) return;
  if (!table && tid == 0) s_tile = atomicAdd(&header[kHdrTicket0 + pass], 1u);
  // after a look-back that gave up (in an earlier pass) the keys are no
  // longer a permutation of the input: this pass stops at once, the whole
  // workgroup together (its successors' bounded waits then give up too).  A
  // plain load: the word was written by an earlier kernel.
  if (tid == 0) s_stop = header[kHdrStop];
  for (int i = tid; i < NW * 256; i += BLOCK) s_match[i] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < 256) s_thist[tid] = 0u;
  __syncthreads();
  if (s_stop) return;
  const uint32_t tile = table ? (uint32_t)xtile : s_tile;
  // uniform: one scalar value for the whole workgroup
  const bool early = !table && __builtin_amdgcn_readfirstlane(header[kHdrEarly0 + pass]) != 0u;
  const uint64_t base = (uint64_t)tile * TILE;

  // load: wave w owns the contiguous run [w*64*E, (w+1)*64*E) of the tile;
  // iteration e reads 64 consecutive keys, so (e, lane) is input order
  // (all loads are issued before any loaded value is used).  Ranks and
  // positions (< 2^13) are kept two per register, and the first pass
  // recomputes its values (the input indices) instead of holding them.
  static_assert(E % 2 == 0 && TILE <= 65536, "16-bit packed ranks");
  uint32_t k[E], v[HOLDV ? E : 1], rkp[E / 2];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t idx = base + (uint64_t)wid * (kWave * E) + (uint64_t)e * kWave + lane;
    const bool valid = idx < n;
    if (MODE == 0) {
      k[e] = valid ? a_bits[idx] : 0u;
      if (PAY) v[HOLDV ? e : 0] = valid ? pay[idx] : 0u;
    } else {
      const uint2 kv = valid ? kvin[idx] : make_uint2(0xFFFFFFFFu, 0u);
      k[e] = kv.x;
      v[HOLDV ? e : 0] = kv.y;
    }
  }
  if (MODE == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t idx = base + (uint64_t)wid * (kWave * E) + (uint64_t)e * kWave + lane;
      k[e] = idx < n ? float_to_key(k[e]) : 0xFFFFFFFFu;
    }
  }
  // With a spread-out digit, the tile's counts first: published before the
  // ranking, they reach successors' look-backs sooner.
  if (early) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t idx = base + (uint64_t)wid * (kWave * E) + (uint64_t)e * kWave + lane;
      if (idx < n) atomicAdd(&s_thist[(k[e] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256 && publish)
      store_agent(status + (uint64_t)tile * 256 + tid,
                  Status<ST>::pack(tile == 0 ? kFlagInclusive : kFlagAggregate, s_thist[tid]));
  }
  // stable rank within the wave's run: earlier iterations first, then lower
  // lanes.  The lanes sharing a digit are found by each lane OR-ing its bit
  // into the digit's mask and reading the mask back (LDS instructions of one
  // wave complete in order, so the read sees every lane's OR of this
  // iteration); the lowest such lane then clears the mask and advances the
  // count.
  uint4* my = s_match + wid * 256;
  const unsigned long long lanebit = 1ull << lane;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t idx = base + (uint64_t)wid * (kWave * E) + (uint64_t)e * kWave + lane;
    const bool valid = idx < n;
    // (keeps the compiler from computing every iteration's digit up front)
    asm volatile("" : "+v"(k[e])::"memory");
    const uint32_t d = (k[e] >> shift) & 255u;
    if (valid)
      __hip_atomic_fetch_or(reinterpret_cast<unsigned long long*>(&my[d]), lanebit, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint4 ent = my[d];
    const uint64_t peers = ((uint64_t)ent.y << 32) | ent.x;
    const uint32_t r = lanes_below(peers);
    const uint32_t next = ent.z + (uint32_t)__popcll(peers);
    if (e % 2 == 0)
      rkp[e / 2] = ent.z + r;
    else
      rkp[e / 2] |= (ent.z + r) << 16;
    asm volatile("" : "+v"(rkp[e / 2]));  // packed now, not at its distant use
    if (valid && r == 0) {
      reinterpret_cast<uint64_t*>(&my[d])[0] = 0ull;
      reinterpret_cast<uint32_t*>(&my[d])[2] = next;
    }
  }
  __syncthreads();

  // per digit (threads 0..255): offsets of each wave inside the tile's digit
  // run, the tile's count, and the inclusive scan of counts over digit values
  const int d = tid & 255;
  const bool digit_owner = tid < 256;
  uint32_t cnt = 0, x = 0;
  if (digit_owner) {
    for (int w = 0; w < NW; ++w) {
      const uint32_t c = s_match[w * 256 + d].z;
      s_whist[w][d] = cnt;
      cnt += c;
    }
    x = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t t = __shfl_up(x, off);
      if (lane >= off) x += t;
    }
    if (lane == kWave - 1) s_wsum[wid] = x;
  }
  // publish this tile's count, then look back for the exclusive prefix:
  // each round reads up to kLookback predecessors at once and consumes them
  // newest first until an inclusive prefix (or a not-yet-published tile)
  uint32_t excl = 0;
  if (table) {
    if (digit_owner) excl = bpre[((uint64_t)(tile >> 1) / chunks_per_block) * 256 + d] + tcount[(uint64_t)tile * 256 + d];
  } else if (digit_owner && (d < 255 ? digit_start[d + 1] : (uint32_t)n) != digit_start[d]) {
    // (a digit value no key has needs no prefix: its owner neither publishes
    // nor looks back, which spares most of the status traffic of a pass
    // whose digit takes few values)
    ST* my = status + (uint64_t)tile * 256 + d;
    if (!early && publish) store_agent(my, Status<ST>::pack(tile == 0 ? kFlagInclusive : kFlagAggregate, cnt));
    if (tile > 0) {
      int64_t t = (int64_t)tile - 1;
      uint32_t spins = 0;
      bool done = false;
      while (!done) {
        ST w[kLookback];
#pragma unroll
        for (int i = 0; i < kLookback; ++i)
          w[i] = (t - i >= 0) ? load_agent(status + (uint64_t)(t - i) * 256 + d) : Status<ST>::pack(kFlagInclusive, 0);
        int used = 0;
#pragma unroll
        for (int i = 0; i < kLookback; ++i) {
          if (done || used < i) continue;  // stopped earlier in this window
          const uint32_t f = Status<ST>::flag(w[i]);
          if (f == 0) continue;            // not published yet: re-read from here
          excl += Status<ST>::value(w[i]);
          used = i + 1;
          if (f == kFlagInclusive) done = true;
        }
        if (!done) {
          t -= used;
          if (used == 0) {
            if (++spins > spin_limit) {
              atomicOr(&header[kHdrFlags], kFlagWatchdog);
              atomicOr(&header[kHdrStop], 1u);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
      }
      if (publish) store_agent(my, Status<ST>::pack(kFlagInclusive, excl + cnt));
    }
  }
  __syncthreads();
  if (digit_owner) {
    uint32_t pre = 0;
    for (int i = 0; i < wid; ++i) pre += s_wsum[i];
    const uint32_t dstart = pre + x - cnt;
    // s_whist[w][d] becomes the tile-local start of wave w's keys of digit d
    for (int w = 0; w < NW; ++w) s_whist[w][d] += dstart;
    s_gbase[d] = digit_start[d] + excl - dstart;  // modular: gbase + local index >= 0
    if (r_dstart != nullptr) {
      r_dstart[(uint64_t)tile * 256 + d] = (uint16_t)dstart;
      r_gbase[(uint64_t)tile * 256 + d] = digit_start[d] + excl - dstart;
    }
  }
  __syncthreads();

  // place the keys in LDS in digit order (stable) and write them out, one
  // half of the tile's sorted order at a time (the staging buffer holds half a
  // tile, which keeps three 512-thread or four 256-thread blocks resident per
  // CU).  All table reads are
  // issued before the LDS writes, and the route's global stores come after
  // them so that no LDS write waits on a store.
  const uint64_t rem = n - base;
  const uint32_t count = rem < (uint64_t)TILE ? (uint32_t)rem : (uint32_t)TILE;
  const uint32_t first = (uint32_t)(wid * (kWave * E) + lane);  // tile-local index at e = 0
  // (the empty asm makes the keys opaque here, so that the digits computed
  // during the ranking are recomputed rather than held in registers across
  // the look-back)
#pragma unroll
  for (int e = 0; e < E; ++e) asm volatile("" : "+v"(k[e]));
  uint32_t posp[E / 2];
#pragma unroll
  for (int e = 0; e < E; e += 2) {
    const uint32_t p0 = s_whist[wid][(k[e] >> shift) & 255u] + (rkp[e / 2] & 0xFFFFu);
    const uint32_t p1 = s_whist[wid][(k[e + 1] >> shift) & 255u] + (rkp[e / 2] >> 16);
    posp[e / 2] = p0 | (p1 << 16);
  }
  auto pos_of = [&](int e) -> uint32_t { return (e % 2 == 0) ? (posp[e / 2] & 0xFFFFu) : (posp[e / 2] >> 16); };
  auto val_of = [&](int e) -> uint32_t {
    return HOLDV ? v[HOLDV ? e : 0] : (uint32_t)(base + first + (uint32_t)(e * kWave));
  };
  constexpr uint32_t HALF = TILE / 2;
  constexpr int kOutSteps = HALF / BLOCK;  // slots per thread and half
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = (uint32_t)h * HALF;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (first + (uint32_t)(e * kWave) < count && pos_of(e) - lo < HALF) s_kv[pos_of(e) - lo] = make_uint2(k[e], val_of(e));
    }
    if (h == 0 && r_lpos != nullptr) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (first + (uint32_t)(e * kWave) < count) r_lpos[base + first + (uint32_t)(e * kWave)] = (uint16_t)pos_of(e);
    }
    __syncthreads();
    // consecutive threads write consecutive slots of a digit's run, in
    // batches whose LDS reads are all issued before their stores
    constexpr int kOutBatch = 4;
    static_assert(kOutSteps % kOutBatch == 0, "write-out batches");
#pragma unroll
    for (int j0 = 0; j0 < kOutSteps; j0 += kOutBatch) {
      uint2 kv[kOutBatch];
      uint32_t o[kOutBatch];
#pragma unroll
      for (int j = 0; j < kOutBatch; ++j) kv[j] = s_kv[(j0 + j) * BLOCK + tid];  // slots past count: stale
#pragma unroll
      for (int j = 0; j < kOutBatch; ++j)
        o[j] = s_gbase[(kv[j].x >> shift) & 255u] + lo + (uint32_t)((j0 + j) * BLOCK + tid);
#pragma unroll
      for (int j = 0; j < kOutBatch; ++j) {
        const uint32_t i = lo + (uint32_t)((j0 + j) * BLOCK + tid);
        // o < n holds for consistent counts; it is checked so nothing is ever written out of range
        if (i < count && (uint64_t)o[j] < n) {
          if (MODE == 2) {
            const uint32_t key = kv[j].x, val = kv[j].y;
            if (PAY)
              kout[o[j]] = key_to_float_bits(key);
            else
              kout[o[j]] = (key == kKeyPlusZero && (uint64_t)val < n) ? a_bits[val] : key_to_float_bits(key);
            vout[o[j]] = val;
          } else {
            kvout[o[j]] = kv[j];
          }
        }
      }
    }
    if (h == 0) __syncthreads();  // the second half reuses the staging buffer
  }
}

// ------------------------------------------------------------------ host side
// pay: NULL (pass 4 writes the permutation to perm) or n payload words that
// ride along with the keys (pass 4 writes them, sorted, to perm).
// table: the first pass takes its offsets from the histogram's tables
// (tcount and the scanned block sums, cpb chunks per histogram block).
// Forced stall (failure-path tests): LAPLEX_DEBUG_STALL=<k> in the
// environment makes the look-back passes publish nothing and give up after
// k spins, so every look-back wait ends at its limit, the watchdog flag is
// raised and laplex_status_poll reports a stall; every kernel still exits.
static uint32_t debug_stall_spins() {
  const char* e = std::getenv("LAPLEX_DEBUG_STALL");
  if (!e || !*e) return 0;
  const unsigned long v = std::strtoul(e, nullptr, 10);
  return (uint32_t)std::min<unsigned long>(v, kSpinLimit);
}

template <typename ST, int TILE>
static hipError_t launch_sort_passes(const SortWorkspace& w, const float* a, uint64_t n, float* a_sorted, uint32_t* perm,
                                     const SortRoute* route, const uint32_t* pay, bool table, uint64_t cpb,
                                     hipStream_t s, bool debug) {
  const uint32_t dbg = debug ? debug_stall_spins() : 0u;
  const uint32_t spin_limit = dbg ? dbg : kSpinLimit;
  const bool publish = dbg == 0;
  const uint32_t* a_bits = reinterpret_cast<const uint32_t*>(a);
  const uint64_t tiles = (n + TILE - 1) / TILE;
  ST* st = reinterpret_cast<ST*>(w.status);
  const uint2* src = nullptr;
  for (int p = 0; p < 4; ++p) {
    ST* stp = st + (uint64_t)p * tiles * 256;
    uint2* dst = (p == 3) ? nullptr : w.kv[p & 1];
    uint32_t* fk = (p == 3) ? reinterpret_cast<uint32_t*>(a_sorted) : nullptr;
    uint32_t* fv = (p == 3) ? perm : nullptr;
    uint16_t* rl = route ? route->lpos[p] : nullptr;
    uint16_t* rd = route ? route->dstart[p] : nullptr;
    uint32_t* rg = route ? route->gbase[p] : nullptr;
    const dim3 grid((unsigned)tiles), grid0((unsigned)xcd_blocks(tiles));
#define LAPLEX_PASS(MODE, PAY, NAME)                                                                                  \
  LAPLEX_LAUNCH(NAME, n, s,                                                                                          \
                (k_onesweep<MODE, ST, PAY, TILE><<<(MODE == 0 && table ? grid0 : grid), dim3(sort_block(MODE, TILE)), 0, s>>>( \
                    src, dst, fk, fv, a_bits, stp, w.header, p, w.offsets + p * 256, n, rl, rd, rg, pay,                \
                    MODE == 0 && table ? w.tcount : nullptr, w.gsum, cpb, spin_limit, publish)))
    if (p == 0 && pay)
      LAPLEX_PASS(0, true, route ? "k_onesweep_first_pay_routed" : "k_onesweep_first_pay");
    else if (p == 0)
      LAPLEX_PASS(0, false, route ? "k_onesweep_first_routed" : "k_onesweep_first");
    else if (p == 3 && pay)
      LAPLEX_PASS(2, true, route ? "k_onesweep_last_pay_routed" : "k_onesweep_last_pay");
    else if (p == 3)
      LAPLEX_PASS(2, false, route ? "k_onesweep_last_routed" : "k_onesweep_last");
    else
      LAPLEX_PASS(1, false, route ? "k_onesweep_mid_routed" : "k_onesweep_mid");
#undef LAPLEX_PASS
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    src = dst;
  }
  return hipSuccess;
}

size_t sort_status_bytes(uint64_t n) {
  const uint64_t tiles = sort_tiles_alloc(n);
  const size_t word = (n <= (1ull << 30)) ? 4 : 8;
  return (size_t)(4 * tiles * 256) * word;
}

static hipError_t sort_impl(const SortWorkspace& w, const float* a, uint64_t n, float* a_sorted, uint32_t* perm,
                            const SortRoute* route, const uint32_t* pay, hipStream_t s, bool debug) {
  if (n == 0) return hipSuccess;
  // clear the header, histograms and look-back status with a fill kernel
  const uint64_t clear_words = (uint64_t)(kSortHeaderBytes / 4) + sort_status_bytes(n) / 4;
  const unsigned fill_blocks = (unsigned)std::min<uint64_t>((clear_words + 255) / 256, 4096);
  LAPLEX_LAUNCH("k_fill_u32", clear_words, s, k_fill_u32<<<fill_blocks, 256, 0, s>>>(w.header, clear_words, 0u));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint64_t chunk = (uint64_t)kHistBlock * kHistItems;
  const uint64_t nchunks = (n + chunk - 1) / chunk;
  const uint64_t hist_blocks = std::min<uint64_t>(nchunks, kHistMaxBlocks);
  const uint64_t cpb = (nchunks + hist_blocks - 1) / hist_blocks;
  LAPLEX_LAUNCH("k_sort_hist", n, s,
                k_sort_hist<<<(unsigned)hist_blocks, kHistBlock, 0, s>>>(reinterpret_cast<const uint32_t*>(a), n, w.hist,
                                                                         w.header, w.tcount, w.gsum, cpb));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // small sorts keep the first pass's look-back; the tables count keys per
  // 8192-key tile, so small tiles always look back
  const bool small = sort_tile(n) == (uint32_t)kSortTileSmall;
  const bool table = !small && sort_tiles(n) >= kTableMinTiles;
  LAPLEX_LAUNCH("k_sort_offsets", 1024, s,
                k_sort_offsets<<<1, kScanThreads, 0, s>>>(w.hist, w.offsets, w.header, w.gsum, table ? hist_blocks : 0));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (small) return launch_sort_passes<uint32_t, kSortTileSmall>(w, a, n, a_sorted, perm, route, pay, false, cpb, s, debug);
  if (n <= (1ull << 30)) return launch_sort_passes<uint32_t, kSortTile>(w, a, n, a_sorted, perm, route, pay, table, cpb, s, debug);
  return launch_sort_passes<uint64_t, kSortTile>(w, a, n, a_sorted, perm, route, pay, table, cpb, s, debug);
}

hipError_t sort_anchors(const SortWorkspace& w, const float* a, uint64_t n, float* a_sorted, uint32_t* perm,
                        const SortRoute* route, hipStream_t s, bool debug_stall) {
  return sort_impl(w, a, n, a_sorted, perm, route, nullptr, s, debug_stall);
}

hipError_t sort_anchors_payload(const SortWorkspace& w, const float* a, const float* x, uint64_t n, float* a_sorted,
                                float* x_sorted, const SortRoute* route, hipStream_t s) {
  return sort_impl(w, a, n, a_sorted, reinterpret_cast<uint32_t*>(x_sorted), route, reinterpret_cast<const uint32_t*>(x), s,
                   false);
}

}  // namespace laplex

namespace laplex {
hipError_t fill_zero_u32(void* p, uint64_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<uint64_t>((words + 255) / 256, 4096);
  LAPLEX_LAUNCH("k_zero_rows", words, s, k_fill_u32<<<blocks, 256, 0, s>>>(static_cast<uint32_t*>(p), words, 0u));
  return hipGetLastError();
}
}  // namespace laplex
