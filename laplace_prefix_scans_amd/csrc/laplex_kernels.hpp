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
int prof_begin(hipStream_t s);
void prof_end(int slot, const char* name, hipStream_t s);
#define LAPLEX_LAUNCH(NAME, STREAM, ...)                \
  do {                                                  \
    const int prof_slot_ = ::laplex::prof_begin(STREAM); \
    __VA_ARGS__;                                        \
    ::laplex::prof_end(prof_slot_, (NAME), (STREAM));   \
  } while (0)

// ------------------------------------------------------------------ sort
constexpr int kSortBlock = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortBlock * kSortItems;

// header words of the sort workspace
constexpr int kHdrFlags = 0;    // sticky error bits (below)
constexpr int kHdrTicket0 = 1;  // one tile ticket per radix pass (4 words)
constexpr uint32_t kFlagNonFinite = 1u, kFlagWatchdog = 2u;
constexpr size_t kSortHeaderBytes = 16384;  // control words, 4x256 histograms, 4x256 offsets
constexpr size_t kSortHistOffset = 1024;
constexpr size_t kSortOffsOffset = 1024 + 4096;

struct SortWorkspace {
  uint32_t* header;   // kSortHeaderBytes, followed directly by the status words
  uint32_t* hist;     // [4][256]
  uint32_t* offsets;  // [4][256]
  void* status;       // [4][tiles][256] u32 (n <= 2^30) or u64
  uint32_t* keys[2];  // ping-pong key buffers, n each
  uint32_t* vals[2];  // ping-pong value buffers, n each
};

size_t sort_status_bytes(uint64_t n);
hipError_t sort_anchors(const SortWorkspace& w, const float* a, uint64_t n, float* a_sorted, uint32_t* perm, hipStream_t s);

// ------------------------------------------------------------------ apply
constexpr int kApplyBlock = 256;
// values per thread: E items x CC columns = 16
constexpr int apply_items(int cc) { return cc >= 16 ? 1 : 16 / cc; }
constexpr int apply_tile(int cc) { return kApplyBlock * apply_items(cc); }

// column chunk: the largest of 8, 4, 2, 1 that divides m
inline uint32_t column_chunk(uint32_t m) { return (m % 8 == 0) ? 8 : (m % 4 == 0) ? 4 : (m % 2 == 0) ? 2 : 1; }

struct ApplyWorkspace {
  float* xs;       // gathered inputs in sorted order (rows x m)
  float* phs;      // gathered input phases in sorted order (phased)
  float* bf;       // [tiles][M] forward tile aggregates
  float* bb;       // [tiles][M] backward tile aggregates
  float* cf;       // [tiles][M] forward carry into each tile
  float* cb;       // [tiles][M] backward carry into each tile
  float2* tanch;   // [tiles] (first, last) anchor of each tile
  uint2* tsplit;   // [tiles+1] merge-path split (a index, b index) at each tile start (general)
};

enum class Variant { Sym, Phased };

hipError_t apply_sym(const ApplyWorkspace& w, Variant var, const float* a_s, const uint32_t* perm, const float* phi, uint64_t n,
                     uint32_t m, const float* x, float* y, hipStream_t s);
hipError_t apply_general(const ApplyWorkspace& w, Variant var, const float* a_s, const uint32_t* perm_a, const float* phi,
                         uint64_t n, const float* b_s, const uint32_t* perm_b, const float* psi, uint64_t k, uint32_t m,
                         const float* x, float* y, hipStream_t s);

// tile count and summary width of an apply
inline uint64_t apply_tiles(uint64_t len, uint32_t m, Variant var) {
  const uint32_t c = column_chunk(m);
  const int cc = (var == Variant::Phased) ? 2 * (int)c : (int)c;
  const uint64_t tile = (uint64_t)apply_tile(cc);
  return (len + tile - 1) / tile;
}

}  // namespace laplex
