// Host-visible launch interface of the LAPLEX kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "laplex_device.hpp"

namespace laplex {

// ------------------------------------------------------------------ opt-in launch profiler
// When enabled through laplex_profile_begin, each kernel launch is bracketed
// by two hipEvents recorded on its stream; otherwise these are no-ops.
// UNITS is the number of elements (rows) the launch processes.
int prof_begin(hipStream_t s);
void prof_end(int slot, const char* name, uint64_t units, hipStream_t s);
#define LAPLEX_LAUNCH(NAME, UNITS, STREAM, ...)                  \
  do {                                                           \
    const int prof_slot_ = ::laplex::prof_begin(STREAM);         \
    __VA_ARGS__;                                                 \
    ::laplex::prof_end(prof_slot_, (NAME), (UNITS), (STREAM));   \
  } while (0)

// ------------------------------------------------------------------ sort
// Sort tiles of 8192 keys.  The first pass (offsets from the histogram's
// tables, no look-back) runs 512 threads x 16 keys; the passes that look back
// run 256 threads x 32 keys, so that four tiles share a CU and more of their
// look-back waits overlap.  Sorts of at most kSmallSortMax keys use tiles of
// 2048 keys (256 threads x 8 keys in every pass): with few tiles a pass lasts
// about as long as one tile, and a quarter of the tile takes about 60 % of
// the time.  The tile size is a function of n alone, so a sort and every
// later use of its route agree on it.  The route kernels move tiles with 512
// threads.
constexpr int kSortTile = 8192;
constexpr int kSortTileSmall = 2048;
constexpr uint64_t kSmallSortMax = 1u << 17;
constexpr int sort_block(int mode, int tile) { return mode == 0 && tile == kSortTile ? 512 : 256; }
constexpr int kRouteBlock = 512;
inline uint32_t sort_tile(uint64_t n) { return n <= kSmallSortMax ? (uint32_t)kSortTileSmall : (uint32_t)kSortTile; }

// header words of the sort workspace
constexpr int kHdrFlags = 0;    // sticky error bits (below)
constexpr int kHdrTicket0 = 1;  // one tile ticket per radix pass (4 words)
// per radix pass: 1 when tiles publish their counts before ranking (4 words;
// a cache line of their own, away from the tickets every workgroup increments)
constexpr int kHdrEarly0 = 64;
// set (with the watchdog flag) when a look-back gives up; read by every tile
// of the later passes, so it too has a cache line of its own
constexpr int kHdrStop = 128;
constexpr uint32_t kFlagNonFinite = 1u, kFlagWatchdog = 2u;
constexpr size_t kSortHeaderBytes = 16384;  // control words, 4x256 histograms, 4x256 offsets
constexpr size_t kSortHistOffset = 1024;
constexpr size_t kSortOffsOffset = 1024 + 4096;

struct SortWorkspace {
  uint32_t* header;   // kSortHeaderBytes, followed directly by the status words
  uint32_t* hist;     // [4][256]
  uint32_t* offsets;  // [4][256]
  void* status;       // [4][tiles][256] u32 (n <= 2^30) or u64
  uint2* kv[2];       // ping-pong buffers of (key, value) pairs, n each
  uint32_t* tcount;   // [tiles][256] first-pass digit counts of the tiles before each tile in its histogram block's range
  uint32_t* gsum;     // [kHistMaxBlocks][256] per histogram block: its range's digit counts, then their exclusive prefix
};
inline uint64_t sort_tiles(uint64_t n) { return (n + sort_tile(n) - 1) / sort_tile(n); }
// Tiles the per-tile arrays (status words, first-pass counts, route tables)
// are laid out for: the sort's own count, but past the switch to 8192-key
// tiles never fewer than the 64 of a sort of kSmallSortMax keys, so that
// every size grows with n and a workspace or route sized for n serves every
// smaller n.
inline uint64_t sort_tiles_alloc(uint64_t n) {
  const uint64_t t = sort_tiles(n), at_switch = kSmallSortMax / kSortTileSmall;
  return n <= kSmallSortMax || t >= at_switch ? t : at_switch;
}
constexpr int kHistMaxBlocks = 256;  // workgroups of the histogram read (rows of gsum)

// Route of a sort: for every radix pass, the tile-local sorted position of
// each element of the pass's input, and per tile the start of each digit's
// run in that order and its global position.  With it a payload can be moved
// between original and sorted order by the same run-coalesced passes the
// sort made (forward: scatter in runs; inverse: gather in runs).
struct SortRoute {
  uint16_t* lpos[4];    // [n]
  uint16_t* dstart[4];  // [tiles][256]
  uint32_t* gbase[4];   // [tiles][256] run position minus local start (mod 2^32)
};
size_t route_bytes(uint64_t n);
SortRoute carve_route(const void* base, uint64_t n);

size_t sort_status_bytes(uint64_t n);
// debug_stall: honour LAPLEX_DEBUG_STALL (only the standalone sort entry
// point does, so that no apply ever runs on a stalled sort's outputs).
hipError_t sort_anchors(const SortWorkspace& w, const float* a, uint64_t n, float* a_sorted, uint32_t* perm,
                        const SortRoute* route, hipStream_t s, bool debug_stall = false);
// The same sort with x (n floats, original order) carried along as the
// value of each key in place of its index: writes x in sorted order to
// x_sorted, and no permutation (the route, if given, still records the
// passes).  -0.0 anchors come out as +0.0.
hipError_t sort_anchors_payload(const SortWorkspace& w, const float* a, const float* x, uint64_t n, float* a_sorted,
                                float* x_sorted, const SortRoute* route, hipStream_t s);

// Move rows of W floats through the sort's passes: forward (original ->
// sorted order) or inverse (sorted -> original).  t0, t1: scratch, n rows each.
hipError_t route_forward(const SortRoute& r, uint64_t n, uint32_t W, const float* in, float* out, float* t0, float* t1,
                         hipStream_t s);
hipError_t route_inverse(const SortRoute& r, uint64_t n, uint32_t W, const float* in, float* out, float* t0, float* t1,
                         hipStream_t s);
constexpr uint32_t kRouteMaxCols = 4;
// Two arrays of n floats moved together as interleaved rows of two, original
// order -> sorted (out: n x 2).  t0, t1: scratch of n x 2 floats each.
hipError_t route_forward_pair(const SortRoute& r, uint64_t n, const float* in0, const float* in1, float* out, float* t0,
                              float* t1, hipStream_t s);

// ------------------------------------------------------------------ apply
// Tile shape for CC injected columns: E consecutive items per thread (the
// single-column cases load them as one float4/float2), threads per block.
constexpr int apply_items(int cc) { return cc == 1 ? 4 : cc == 2 ? 2 : cc >= 16 ? 1 : 16 / cc; }
constexpr int apply_block(int cc) { return cc <= 2 ? 1024 : 256; }
constexpr int apply_tile(int cc) { return apply_block(cc) * apply_items(cc); }

// column chunk: the largest of 8, 4, 2, 1 that divides m
inline uint32_t column_chunk(uint32_t m) { return (m % 8 == 0) ? 8 : (m % 4 == 0) ? 4 : (m % 2 == 0) ? 2 : 1; }
// phased applies scan a cos and a sin column per input column: chunks of at
// most 4 (8 scanned columns) keep a tile's state in registers
inline uint32_t phased_chunk(uint32_t m) { const uint32_t c = column_chunk(m); return c > 4 ? 4 : c; }

struct ApplyWorkspace {
  float* xs;       // gathered inputs in sorted order (rows x m)
  float* phs;      // gathered input phases in sorted order (phased)
  float* zs;       // outputs in sorted order before the inverse route (rows_out x m)
  float* phas;     // output phases in sorted order (phased general with a route)
  float* t0;       // route scratch (max rows x m)
  float* t1;       // route scratch (max rows x m)
  float* bf;       // [tiles][M] forward tile aggregates
  float* bb;       // [tiles][M] backward tile aggregates
  float* cf;       // [tiles][M] forward carry into each tile
  float* cb;       // [tiles][M] backward carry into each tile
  float2* tanch;   // [tiles] (first, last) anchor of each tile
  float* gbf;      // [groups][M] group aggregates and carries (groups = tiles / 1024, rounded up)
  float* gbb;
  float* gcf;
  float* gcb;
  float2* ganch;   // [groups]
  uint2* tsplit;   // [tiles+1] merge-path split (a index, b index) at each tile start (general)
};

enum class Variant { Sym, Phased };

// route / route_a / route_b may be null (then x and y move by index).
hipError_t apply_sym(const ApplyWorkspace& w, Variant var, const float* a_s, const uint32_t* perm, const SortRoute* route,
                     const float* phi, uint64_t n, uint32_t m, const float* x, float* y, hipStream_t s);
// Symmetric apply, one column, with w.xs already holding x in sorted order
// (from sort_anchors_payload): scans, then y back along the route.
hipError_t apply_sym_presorted(const ApplyWorkspace& w, const float* a_s, const SortRoute& route, uint64_t n, float* y,
                               hipStream_t s);
// General operator from unsorted output anchors a (n) and sorted inputs
// b_s (k >= 1, sort handle perm_b): the scans run over b alone (Fi into fo,
// U into uo, k x m each; for one column also a table in fu of
// search_table_bytes(k): (Fi_{q-1}, U_q) per interval, k + 1, then the
// search's sample tree) and each output searches its interval in b_s; y in
// the original order of a.  Non-finite a raise kFlagNonFinite in header.
constexpr int kSearchTree = 8192;  // slots of the search's sample tree (a power of two)
inline size_t search_table_bytes(uint64_t k) { return (size_t)(k + 1) * 8 + 256 + (size_t)kSearchTree * 4; }
inline float* search_tree(float2* fu, uint64_t k) {
  return reinterpret_cast<float*>((reinterpret_cast<uintptr_t>(fu + k + 1) + 255) & ~uintptr_t(255));
}
hipError_t apply_general_search(const ApplyWorkspace& w, float* fo, float* uo, float2* fu, const float* a, uint64_t n, const float* b_s,
                                const uint32_t* perm_b, uint64_t k, uint32_t m, const float* x, float* y, uint32_t* header,
                                hipStream_t s);
hipError_t apply_general(const ApplyWorkspace& w, Variant var, const float* a_s, const uint32_t* perm_a, const SortRoute* route_a,
                         const float* phi, uint64_t n, const float* b_s, const uint32_t* perm_b, const SortRoute* route_b,
                         const float* psi, uint64_t k, uint32_t m, const float* x, float* y, hipStream_t s);

// Backward of the symmetric operator: dx = K g and the anchor gradient da.
// Uses an apply workspace whose summary width is M = 4m (x and g, each with
// the kernel's decay and with the tie decay); zs holds dx in sorted order.
struct BackwardWorkspace {
  ApplyWorkspace w;
  float* gs;   // upstream gradient gathered into sorted(-a) order (n x m)
  float* das;  // anchor gradient in sorted(-a) order (n)
  float* dbs;  // column-anchor gradient in sorted-b order (k; general only)
  float* dphs;   // phase gradient in sorted(-a) order (n; phased only)
  float* dpsis;  // column-phase gradient in sorted-b order (k; general phased only)
};
// xs_sorted: x already in sorted order (n x m, e.g. kept by a forward apply);
// then x is not read and only g is moved.
hipError_t backward_sym(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm, const SortRoute* route,
                        uint64_t n, uint32_t m, const float* x, const float* g, float* dx, float* da, hipStream_t s,
                        const float* xs_sorted = nullptr);

// Backward of the symmetric phased operator: dx (n x m), da, dphi (n).  Scans
// four columns per input column (cos/sin phase times x and g) under both
// decays: summary width M = 8m, tiles of the 4-column shape; xs, gs, phs hold
// x, g, phi in sorted order, zs dx in sorted order.
hipError_t backward_phased(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm, const SortRoute* route,
                           const float* phi, uint64_t n, uint32_t m, const float* x, const float* g, float* dx, float* da,
                           float* dphi, hipStream_t s);
constexpr int kPbwdChunk = 1;  // input columns per pass of the phased backward
inline uint64_t phased_backward_tiles(uint64_t n, uint32_t m) {
  (void)m;
  const uint64_t tile = (uint64_t)apply_tile(4 * kPbwdChunk);
  return (n + tile - 1) / tile;
}

// Backward of the general phased operator (rows a, phi; columns b, psi):
// dx (k x m), da, dphi (n), db, dpsi (k); one merged two-decay scan of four
// columns per input column (M = 8m).  xs / phs: x and psi in sorted-b order;
// gs / phas: g and phi in sorted-a order; zs: dx in sorted-b order.  Requires
// n, k >= 1.
hipError_t backward_phased_general(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm_a,
                                   const SortRoute* route_a, const float* phi, uint64_t n, const float* b_s,
                                   const uint32_t* perm_b, const SortRoute* route_b, const float* psi, uint64_t k, uint32_t m,
                                   const float* x, const float* g, float* dx, float* da, float* db, float* dphi, float* dpsi,
                                   hipStream_t s);

// Backward of the general operator (rows a, n; columns b, k): dx = K^T g
// (k x m), da (n), db (k).  One scan over the merge of a and b with summary
// width M = 4m; xs holds x in sorted-b order, gs g in sorted-a order, zs dx in
// sorted-b order.  Requires n, k >= 1.
hipError_t backward_general(const BackwardWorkspace& bw, const float* a_s, const uint32_t* perm_a, const SortRoute* route_a,
                            uint64_t n, const float* b_s, const uint32_t* perm_b, const SortRoute* route_b, uint64_t k,
                            uint32_t m, const float* x, const float* g, float* dx, float* da, float* db, hipStream_t s);

// Weighted Gram matrix M = A diag(D) A^T (A = LAPLEX(a, b)): rows
// [r0, r0 + rc) of M in the original order of a, written to M[(p - r0) * ldm + q].
// Uses the merged-scan part of an apply workspace (tiles of the merge of n + k
// anchors, one summary column) plus the families below.  Requires n >= 1; with
// k == 0 it writes zeros.
struct GramWorkspace {
  ApplyWorkspace w;
  float* a2;     // doubled sorted a (n)
  float* b2;     // doubled sorted b (k)
  float* Ds;     // D in sorted-b order (k)
  double* Cpre;  // exclusive prefix sums of Ds (k + 1)
  float* Ao;     // per output anchor, original order: the anchor (n)
  float* Po;     //   P (n)
  float* Qo;     //   Q (n)
  double* Co;    //   C (n)
};
hipError_t gram_weighted(const GramWorkspace& g, const float* a_s, const uint32_t* perm_a, uint64_t n, const float* b_s,
                         const uint32_t* perm_b, uint64_t k, const float* D, uint64_t r0, uint64_t rc, float* M, uint64_t ldm,
                         hipStream_t s);

// tile count and summary width of an apply
inline uint64_t apply_tiles(uint64_t len, uint32_t m, Variant var) {
  const uint32_t c = (var == Variant::Phased) ? phased_chunk(m) : column_chunk(m);
  const int cc = (var == Variant::Phased) ? 2 * (int)c : (int)c;
  const uint64_t tile = (uint64_t)apply_tile(cc);
  return (len + tile - 1) / tile;
}

// Tile shape of the symmetric backward for a chunk of c columns (2c scanned
// columns, x and g).  One column: 512-thread workgroups of 4 items each, so
// two workgroups share a compute unit without spilling and one's loads
// overlap the other's scans.
constexpr int bwd_items(int c) { return c == 1 ? 4 : apply_items(2 * c); }
constexpr int bwd_block(int c) { return c == 1 ? 512 : apply_block(2 * c); }
constexpr int bwd_tile(int c) { return bwd_items(c) * bwd_block(c); }

// tile count of a symmetric backward
inline uint64_t backward_tiles(uint64_t n, uint32_t m) {
  const uint64_t tile = (uint64_t)bwd_tile((int)column_chunk(m));
  return (n + tile - 1) / tile;
}

}  // namespace laplex
