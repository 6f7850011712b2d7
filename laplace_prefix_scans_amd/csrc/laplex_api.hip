// C-ABI entry points: argument checks, workspace layout, launches.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/laplex.h"
#include "laplex_kernels.hpp"

namespace laplex {
hipError_t fill_zero_u32(void* p, uint64_t words, hipStream_t s);
}

namespace {

using namespace laplex;

constexpr uint64_t kMaxLen = 0xFFFFFFFFull;  // uint32 permutations
constexpr uint32_t kMaxCols = 1u << 16;
constexpr uint64_t kGramMaxLen = 65535ull * 1024;  // columns of the Gram fill grid

// Carves 256-byte aligned regions out of a workspace (base 0: sizing only).
struct Carver {
  uintptr_t base;
  size_t off = 0;
  explicit Carver(void* b) : base(reinterpret_cast<uintptr_t>(b)) {}
  template <typename T>
  T* take(size_t bytes) {
    off = (off + 255) & ~size_t(255);
    T* p = reinterpret_cast<T*>(base + off);
    off += bytes;
    return p;
  }
};

SortWorkspace carve_sort(void* ws, uint64_t n) {
  Carver c(ws);
  SortWorkspace w;
  w.header = c.take<uint32_t>(kSortHeaderBytes);
  w.hist = w.header + kSortHistOffset / 4;
  w.offsets = w.header + kSortOffsOffset / 4;
  w.status = c.take<void>(sort_status_bytes(n));  // directly after the header
  for (int i = 0; i < 2; ++i) w.kv[i] = c.take<uint2>(n * 8);
  w.tcount = c.take<uint32_t>(sort_tiles_alloc(n) * 256 * 4);
  w.gsum = c.take<uint32_t>((size_t)kHistMaxBlocks * 256 * 4);
  return w;
}
size_t sort_bytes(uint64_t n) {
  Carver c(nullptr);
  c.take<uint32_t>(kSortHeaderBytes);
  c.take<void>(sort_status_bytes(n));
  for (int i = 0; i < 2; ++i) c.take<uint2>(n * 8);
  c.take<uint32_t>(sort_tiles_alloc(n) * 256 * 4);
  c.take<uint32_t>((size_t)kHistMaxBlocks * 256 * 4);
  return (c.off + 255) & ~size_t(255);
}

// rows_in: length of the gathered input (n symmetric, k general); rows_out:
// outputs (n); len: scanned length.  Buffers for moving x and y along a sort
// route (zs, t0, t1, phas) are laid out when m is small enough for routes.
ApplyWorkspace carve_apply(void* ws, uint64_t rows_in, uint64_t rows_out, uint64_t len, uint32_t m, Variant var, bool general,
                           size_t* total) {
  Carver c(ws);
  ApplyWorkspace w{};
  const uint64_t T = apply_tiles(len, m, var);
  const uint64_t M = (var == Variant::Phased) ? 2ull * m : m;
  const bool ph = var == Variant::Phased;
  w.xs = c.take<float>(rows_in * m * 4);
  w.phs = ph ? c.take<float>(rows_in * 4) : nullptr;
  w.bf = c.take<float>(T * M * 4);
  w.bb = c.take<float>(T * M * 4);
  w.cf = c.take<float>(T * M * 4);
  w.cb = c.take<float>(T * M * 4);
  w.tanch = c.take<float2>(T * 8);
  const uint64_t G = (T + 1023) / 1024;
  w.gbf = c.take<float>(G * M * 4);
  w.gbb = c.take<float>(G * M * 4);
  w.gcf = c.take<float>(G * M * 4);
  w.gcb = c.take<float>(G * M * 4);
  w.ganch = c.take<float2>(G * 8);
  w.tsplit = general ? c.take<uint2>((T + 1) * 8) : nullptr;
  if (m <= kRouteMaxCols) {
    const uint64_t rmax = std::max(rows_in, rows_out);
    w.zs = c.take<float>(rows_out * m * 4);
    w.phas = (ph && general) ? c.take<float>(rows_out * 4) : nullptr;
    w.t0 = c.take<float>(rmax * m * 4);
    w.t1 = c.take<float>(rmax * m * 4);
  }
  if (total) *total = (c.off + 255) & ~size_t(255);
  return w;
}

// Symmetric (k = 0, general false), general, or symmetric phased backward:
// gathered inputs, sorted-order outputs, tile summaries (width 4m, or 8m
// phased) over the n (+ k) scanned elements, and route scratch when m is small
// enough for routes.
BackwardWorkspace carve_backward(void* ws, uint64_t n, uint64_t k, uint32_t m, bool general, size_t* total,
                                 bool phased = false) {
  Carver c(ws);
  BackwardWorkspace bw{};
  ApplyWorkspace& w = bw.w;
  const uint64_t rows_x = general ? k : n;  // rows of x and dx
  const uint64_t T = phased ? phased_backward_tiles(general ? n + k : n, m) : backward_tiles(general ? n + k : n, m);
  const uint64_t M = (phased ? 8ull : 4ull) * m;
  // one symmetric column moves x with g as rows of two
  const uint64_t mp = (!general && !phased && m == 1) ? 2 : m;
  w.xs = c.take<float>(rows_x * mp * 4);
  bw.gs = c.take<float>(n * m * 4);
  w.zs = c.take<float>(rows_x * m * 4);
  bw.das = c.take<float>(n * 4);
  bw.dbs = general ? c.take<float>(k * 4) : nullptr;
  w.phs = phased ? c.take<float>(rows_x * 4) : nullptr;           // phases of x's rows, sorted
  w.phas = (phased && general) ? c.take<float>(n * 4) : nullptr;  // phases of the rows of a, sorted
  bw.dphs = phased ? c.take<float>(n * 4) : nullptr;
  bw.dpsis = (phased && general) ? c.take<float>(k * 4) : nullptr;
  w.bf = c.take<float>(T * M * 4);
  w.bb = c.take<float>(T * M * 4);
  w.cf = c.take<float>(T * M * 4);
  w.cb = c.take<float>(T * M * 4);
  w.tanch = c.take<float2>(T * 8);
  const uint64_t G = (T + 1023) / 1024;
  w.gbf = c.take<float>(G * M * 4);
  w.gbb = c.take<float>(G * M * 4);
  w.gcf = c.take<float>(G * M * 4);
  w.gcb = c.take<float>(G * M * 4);
  w.ganch = c.take<float2>(G * 8);
  w.tsplit = general ? c.take<uint2>((T + 1) * 8) : nullptr;
  if (m <= kRouteMaxCols) {
    const uint64_t rmax = std::max(n, rows_x);
    w.t0 = c.take<float>(rmax * mp * 4);
    w.t1 = c.take<float>(rmax * mp * 4);
  }
  if (total) *total = (c.off + 255) & ~size_t(255);
  return bw;
}

// Weighted Gram: merged-scan tiles of the n + k anchors (one summary column)
// and the per-anchor families.
GramWorkspace carve_gram(void* ws, uint64_t n, uint64_t k, size_t* total) {
  Carver c(ws);
  GramWorkspace g{};
  ApplyWorkspace& w = g.w;
  const uint64_t T = (n + k + apply_tile(1) - 1) / apply_tile(1);
  w.bf = c.take<float>(T * 4);
  w.bb = c.take<float>(T * 4);
  w.cf = c.take<float>(T * 4);
  w.cb = c.take<float>(T * 4);
  w.tanch = c.take<float2>(T * 8);
  const uint64_t G = (T + 1023) / 1024;
  w.gbf = c.take<float>(G * 4);
  w.gbb = c.take<float>(G * 4);
  w.gcf = c.take<float>(G * 4);
  w.gcb = c.take<float>(G * 4);
  w.ganch = c.take<float2>(G * 8);
  w.tsplit = c.take<uint2>((T + 1) * 8);
  g.a2 = c.take<float>(n * 4);
  g.b2 = c.take<float>(k * 4);
  g.Ds = c.take<float>(k * 4);
  g.Cpre = c.take<double>((k + 1) * 8);
  g.Ao = c.take<float>(n * 4);
  g.Po = c.take<float>(n * 4);
  g.Qo = c.take<float>(n * 4);
  g.Co = c.take<double>(n * 8);
  if (total) *total = (c.off + 255) & ~size_t(255);
  return g;
}

// Sort and symmetric apply in one call: the sort workspace first (so that
// laplex_status_poll finds its flags at the start), then the sorted anchors,
// the route and the apply workspace; the permutation only when m != 1.
struct SortSymWorkspace {
  SortWorkspace sort;
  float* a_s;
  uint32_t* perm;
  void* route;
  ApplyWorkspace apply;
};
SortSymWorkspace carve_sort_sym(void* ws, uint64_t n, uint32_t m, size_t* total) {
  Carver c(ws);
  SortSymWorkspace w{};
  char* sort_base = c.take<char>(sort_bytes(n));
  if (ws) w.sort = carve_sort(sort_base, n);
  w.a_s = c.take<float>(n * 4);
  w.perm = m == 1 ? nullptr : c.take<uint32_t>(n * 4);
  w.route = m <= kRouteMaxCols ? c.take<void>(route_bytes(n)) : nullptr;
  char* apply_base = c.take<char>(0);
  size_t apply_total = 0;
  w.apply = carve_apply(ws ? apply_base : nullptr, n, n, n, m, Variant::Sym, false, &apply_total);
  c.off += apply_total;
  if (total) *total = (c.off + 255) & ~size_t(255);
  return w;
}

// Sort of b and the general operator with the scans over b, in one call: the
// sort workspace of b first (so that laplex_status_poll finds its flags at
// the start), b's sort handle, the apply workspace over b, and Fi, U.
struct SortGeneralWorkspace {
  SortWorkspace sort;
  float* b_s;
  uint32_t* perm_b;
  ApplyWorkspace apply;
  float* fo;
  float* uo;
  float2* fu;
};
SortGeneralWorkspace carve_sort_general(void* ws, uint64_t k, uint32_t m, size_t* total) {
  Carver c(ws);
  SortGeneralWorkspace w{};
  char* sort_base = c.take<char>(sort_bytes(k));
  if (ws) w.sort = carve_sort(sort_base, k);
  w.b_s = c.take<float>(k * 4);
  w.perm_b = c.take<uint32_t>(k * 4);
  w.fo = c.take<float>(k * m * 4);
  w.uo = c.take<float>(k * m * 4);
  w.fu = m == 1 ? c.take<float2>(search_table_bytes(k)) : nullptr;
  char* apply_base = c.take<char>(0);
  size_t apply_total = 0;
  w.apply = carve_apply(ws ? apply_base : nullptr, k, k, k, m, Variant::Sym, false, &apply_total);
  c.off += apply_total;
  if (total) *total = (c.off + 255) & ~size_t(255);
  return w;
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlaps(const void* p, size_t pb, const void* q, size_t qb) {
  if (!p || !q || pb == 0 || qb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + pb;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + qb;
  return a0 < b1 && b0 < a1;
}

laplex_status from_hip(hipError_t e) { return e == hipSuccess ? LAPLEX_OK : LAPLEX_ERR_HIP; }

}  // namespace

extern "C" size_t laplex_workspace_bytes(int op, uint64_t n, uint64_t k, uint32_t m) {
  if (n > kMaxLen || k > kMaxLen || m > kMaxCols) return 0;
  if (m == 0) m = 1;
  size_t total = 0;
  switch (op) {
    case LAPLEX_OP_SORT: return sort_bytes(n);
    case LAPLEX_OP_SYM: carve_apply(nullptr, n, n, n, m, Variant::Sym, false, &total); return total;
    case LAPLEX_OP_PHASED: carve_apply(nullptr, n, n, n, m, Variant::Phased, false, &total); return total;
    case LAPLEX_OP_GENERAL: carve_apply(nullptr, k, n, n + k, m, Variant::Sym, true, &total); return total;
    case LAPLEX_OP_PHASED_GENERAL: carve_apply(nullptr, k, n, n + k, m, Variant::Phased, true, &total); return total;
    case LAPLEX_OP_SYM_BACKWARD: carve_backward(nullptr, n, 0, m, false, &total); return total;
    case LAPLEX_OP_GENERAL_BACKWARD: carve_backward(nullptr, n, k, m, true, &total); return total;
    case LAPLEX_OP_GRAM: carve_gram(nullptr, n, k, &total); return total;
    case LAPLEX_OP_PHASED_BACKWARD: carve_backward(nullptr, n, 0, m, false, &total, true); return total;
    case LAPLEX_OP_PHASED_GENERAL_BACKWARD: carve_backward(nullptr, n, k, m, true, &total, true); return total;
    case LAPLEX_OP_SORT_SYM: carve_sort_sym(nullptr, n, m, &total); return total;
    case LAPLEX_OP_SORT_GENERAL: carve_sort_general(nullptr, k, m, &total); return total;
    default: return 0;
  }
}

extern "C" size_t laplex_route_bytes(uint64_t n) {
  if (n > kMaxLen) return 0;
  return route_bytes(n);
}

extern "C" laplex_status laplex_sort_anchors(const float* a, uint64_t n, float* a_sorted, uint32_t* perm, void* route,
                                             size_t route_bytes_, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n == 0) return LAPLEX_OK;
  if (n > kMaxLen) return LAPLEX_ERR_SIZE;
  if (!a || !a_sorted || !perm || !ws) return LAPLEX_ERR_NULL;
  if (misaligned(a, 4) || misaligned(a_sorted, 4) || misaligned(perm, 4) || misaligned(ws, 256) ||
      (route && misaligned(route, 256)))
    return LAPLEX_ERR_ALIGN;
  if (ws_bytes < sort_bytes(n)) return LAPLEX_ERR_WORKSPACE;
  if (route && route_bytes_ < route_bytes(n)) return LAPLEX_ERR_WORKSPACE;
  const size_t vb = n * 4;
  if (overlaps(a_sorted, vb, a, vb) || overlaps(perm, vb, a, vb) || overlaps(a_sorted, vb, perm, vb) ||
      overlaps(a_sorted, vb, ws, ws_bytes) || overlaps(perm, vb, ws, ws_bytes))
    return LAPLEX_ERR_OVERLAP;
  if (route && (overlaps(route, route_bytes_, a, vb) || overlaps(route, route_bytes_, a_sorted, vb) ||
                overlaps(route, route_bytes_, perm, vb) || overlaps(route, route_bytes_, ws, ws_bytes)))
    return LAPLEX_ERR_OVERLAP;
  const SortWorkspace w = carve_sort(ws, n);
  SortRoute r{};
  if (route) r = carve_route(route, n);
  return from_hip(sort_anchors(w, a, n, a_sorted, perm, route ? &r : nullptr, stream, true));
}

extern "C" laplex_status laplex_status_poll(const void* ws, hipStream_t stream) {
  if (!ws) return LAPLEX_ERR_NULL;
  if (hipStreamSynchronize(stream) != hipSuccess) return LAPLEX_ERR_HIP;
  uint32_t flags = 0;
  if (hipMemcpy(&flags, static_cast<const uint32_t*>(ws) + kHdrFlags, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return LAPLEX_ERR_HIP;
  if (flags & kFlagNonFinite) return LAPLEX_ERR_NONFINITE;
  if (flags & kFlagWatchdog) return LAPLEX_ERR_STALLED;
  return LAPLEX_OK;
}

static laplex_status check_apply_common(const float* a_sorted, const uint32_t* perm, uint64_t n, uint32_t m, const float* x,
                                        float* y, void* ws) {
  if (n > kMaxLen) return LAPLEX_ERR_SIZE;
  if (m > kMaxCols) return LAPLEX_ERR_SIZE;
  if (!a_sorted || !perm || !x || !y || !ws) return LAPLEX_ERR_NULL;
  if (misaligned(a_sorted, 4) || misaligned(perm, 4) || misaligned(x, 4) || misaligned(y, 4) || misaligned(ws, 256))
    return LAPLEX_ERR_ALIGN;
  return LAPLEX_OK;
}

extern "C" laplex_status laplex_matvec_sym(const float* a_sorted, const uint32_t* perm, const void* route, uint64_t n, uint32_t m,
                                           const float* x, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n == 0 || m == 0) return LAPLEX_OK;
  laplex_status st = check_apply_common(a_sorted, perm, n, m, x, y, ws);
  if (st != LAPLEX_OK) return st;
  if (route && misaligned(route, 256)) return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_apply(nullptr, n, n, n, m, Variant::Sym, false, &need);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t yb = n * (size_t)m * 4, vb = n * 4;
  if (overlaps(y, yb, x, yb) || overlaps(y, yb, a_sorted, vb) || overlaps(y, yb, perm, vb) || overlaps(y, yb, ws, ws_bytes) ||
      overlaps(y, yb, route, route ? route_bytes(n) : 0))
    return LAPLEX_ERR_OVERLAP;
  const ApplyWorkspace w = carve_apply(ws, n, n, n, m, Variant::Sym, false, nullptr);
  SortRoute r{};
  if (route) r = carve_route(route, n);
  return from_hip(apply_sym(w, Variant::Sym, a_sorted, perm, route ? &r : nullptr, nullptr, n, m, x, y, stream));
}

// ------------------------------------------------------------------ allocation-free variant
// The workspace of laplex_matvec_sym_noalloc: one static array per GPU.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[LAPLEX_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// Device address of the scratch array on the device of `stream` (the current
// device for the null stream).
laplex_status scratch_address(hipStream_t stream, void** out) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return LAPLEX_ERR_HIP;
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return LAPLEX_ERR_HIP;
  if (dev < 0 || dev >= kScratchDevices) return LAPLEX_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return LAPLEX_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return LAPLEX_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LAPLEX_OK;
}
}  // namespace

extern "C" laplex_status laplex_matvec_sym_noalloc(const float* a_sorted, const uint32_t* perm, const void* route, uint64_t n,
                                                   uint32_t m, const float* x, float* y, hipStream_t stream) {
  if (n == 0 || m == 0) return LAPLEX_OK;
  if (n > kMaxLen || m > kMaxCols) return LAPLEX_ERR_SIZE;
  size_t need = 0;
  carve_apply(nullptr, n, n, n, m, Variant::Sym, false, &need);
  if (need > LAPLEX_SCRATCH_BYTES) return LAPLEX_ERR_SCRATCH;
  void* ws = nullptr;
  const laplex_status st = scratch_address(stream, &ws);
  if (st != LAPLEX_OK) return st;
  return laplex_matvec_sym(a_sorted, perm, route, n, m, x, y, ws, LAPLEX_SCRATCH_BYTES, stream);
}

extern "C" laplex_status laplex_sort_matvec_sym(const float* a, uint64_t n, uint32_t m, const float* x, float* y, void* ws,
                                                size_t ws_bytes, hipStream_t stream) {
  if (n == 0 || m == 0) return LAPLEX_OK;
  if (n > kMaxLen || m > kMaxCols) return LAPLEX_ERR_SIZE;
  if (!a || !x || !y || !ws) return LAPLEX_ERR_NULL;
  if (misaligned(a, 4) || misaligned(x, 4) || misaligned(y, 4) || misaligned(ws, 256)) return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_sort_sym(nullptr, n, m, &need);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t yb = n * (size_t)m * 4, vb = n * 4;
  if (overlaps(y, yb, x, yb) || overlaps(y, yb, a, vb) || overlaps(y, yb, ws, ws_bytes) || overlaps(a, vb, ws, ws_bytes) ||
      overlaps(x, yb, ws, ws_bytes))
    return LAPLEX_ERR_OVERLAP;
  const SortSymWorkspace w = carve_sort_sym(ws, n, m, nullptr);
  SortRoute r{};
  if (w.route) r = carve_route(w.route, n);
  hipError_t e;
  if (m == 1) {
    if ((e = sort_anchors_payload(w.sort, a, x, n, w.a_s, w.apply.xs, &r, stream)) != hipSuccess) return from_hip(e);
    return from_hip(apply_sym_presorted(w.apply, w.a_s, r, n, y, stream));
  }
  if ((e = sort_anchors(w.sort, a, n, w.a_s, w.perm, w.route ? &r : nullptr, stream)) != hipSuccess) return from_hip(e);
  return from_hip(apply_sym(w.apply, Variant::Sym, w.a_s, w.perm, w.route ? &r : nullptr, nullptr, n, m, x, y, stream));
}

extern "C" laplex_status laplex_sort_matvec_general(const float* a, uint64_t n, const float* b, uint64_t k, uint32_t m,
                                                    const float* x, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n == 0 || m == 0) return LAPLEX_OK;
  if (n > kMaxLen || k > kMaxLen || m > kMaxCols) return LAPLEX_ERR_SIZE;
  if (!a || !y || !ws || (k > 0 && (!b || !x))) return LAPLEX_ERR_NULL;
  if (misaligned(a, 4) || misaligned(b, 4) || misaligned(x, 4) || misaligned(y, 4) || misaligned(ws, 256))
    return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_sort_general(nullptr, k, m, &need);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t yb = n * (size_t)m * 4, xb = k * (size_t)m * 4;
  if (overlaps(y, yb, a, n * 4) || overlaps(y, yb, b, k * 4) || overlaps(y, yb, x, xb) || overlaps(y, yb, ws, ws_bytes) ||
      overlaps(a, n * 4, ws, ws_bytes) || overlaps(b, k * 4, ws, ws_bytes) || overlaps(x, xb, ws, ws_bytes))
    return LAPLEX_ERR_OVERLAP;
  hipError_t e;
  if (k == 0) {  // no inputs: y = 0, and no stale flags for laplex_status_poll
    if ((e = fill_zero_u32(ws, kSortHeaderBytes / 4, stream)) != hipSuccess) return from_hip(e);
    return from_hip(fill_zero_u32(y, n * (uint64_t)m, stream));
  }
  const SortGeneralWorkspace w = carve_sort_general(ws, k, m, nullptr);
  if ((e = sort_anchors(w.sort, b, k, w.b_s, w.perm_b, nullptr, stream)) != hipSuccess) return from_hip(e);
  return from_hip(apply_general_search(w.apply, w.fo, w.uo, w.fu, a, n, w.b_s, w.perm_b, k, m, x, y, w.sort.header, stream));
}

extern "C" laplex_status laplex_sort_matvec_sym_backward(const void* fwd_ws, size_t fwd_ws_bytes, uint64_t n, uint32_t m,
                                                         const float* g, float* dx, float* da, void* ws, size_t ws_bytes,
                                                         hipStream_t stream) {
  if (n == 0 || m == 0) return LAPLEX_OK;
  if (n > kMaxLen || m > kMaxCols) return LAPLEX_ERR_SIZE;
  if (!fwd_ws || !g || !dx || !da || !ws) return LAPLEX_ERR_NULL;
  if (misaligned(fwd_ws, 256) || misaligned(g, 4) || misaligned(dx, 4) || misaligned(da, 4) || misaligned(ws, 256))
    return LAPLEX_ERR_ALIGN;
  size_t need_f = 0, need = 0;
  carve_sort_sym(nullptr, n, m, &need_f);
  carve_backward(nullptr, n, 0, m, false, &need);
  if (fwd_ws_bytes < need_f || ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t xb = n * (size_t)m * 4, vb = n * 4;
  for (const void* out : {static_cast<const void*>(dx), static_cast<const void*>(da)}) {
    const size_t ob = out == dx ? xb : vb;
    if (overlaps(out, ob, g, xb) || overlaps(out, ob, fwd_ws, fwd_ws_bytes) || overlaps(out, ob, ws, ws_bytes)) return LAPLEX_ERR_OVERLAP;
  }
  if (overlaps(dx, xb, da, vb) || overlaps(ws, ws_bytes, fwd_ws, fwd_ws_bytes) || overlaps(g, xb, ws, ws_bytes))
    return LAPLEX_ERR_OVERLAP;
  // the forward's sorted anchors, permutation (m != 1), route (m <= 4) and
  // x in sorted order (left in its apply workspace)
  const SortSymWorkspace f = carve_sort_sym(const_cast<void*>(fwd_ws), n, m, nullptr);
  SortRoute r{};
  if (f.route) r = carve_route(f.route, n);
  const BackwardWorkspace bw = carve_backward(ws, n, 0, m, false, nullptr);
  return from_hip(backward_sym(bw, f.a_s, f.perm, f.route ? &r : nullptr, n, m, nullptr, g, dx, da, stream, f.apply.xs));
}

extern "C" laplex_status laplex_backward_sym(const float* a_sorted, const uint32_t* perm, const void* route, uint64_t n,
                                             uint32_t m, const float* x, const float* g, float* dx, float* da, void* ws,
                                             size_t ws_bytes, hipStream_t stream) {
  if (n == 0 || m == 0) return LAPLEX_OK;
  laplex_status st = check_apply_common(a_sorted, perm, n, m, x, dx, ws);
  if (st != LAPLEX_OK) return st;
  if (!g || !da) return LAPLEX_ERR_NULL;
  if (misaligned(g, 4) || misaligned(da, 4) || (route && misaligned(route, 256))) return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_backward(nullptr, n, 0, m, false, &need);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t xb = n * (size_t)m * 4, vb = n * 4, rb = route ? route_bytes(n) : 0;
  for (const void* out : {static_cast<const void*>(dx), static_cast<const void*>(da)}) {
    const size_t ob = out == dx ? xb : vb;
    if (overlaps(out, ob, x, xb) || overlaps(out, ob, g, xb) || overlaps(out, ob, a_sorted, vb) || overlaps(out, ob, perm, vb) ||
        overlaps(out, ob, ws, ws_bytes) || overlaps(out, ob, route, rb))
      return LAPLEX_ERR_OVERLAP;
  }
  if (overlaps(dx, xb, da, vb)) return LAPLEX_ERR_OVERLAP;
  const BackwardWorkspace bw = carve_backward(ws, n, 0, m, false, nullptr);
  SortRoute r{};
  if (route) r = carve_route(route, n);
  return from_hip(backward_sym(bw, a_sorted, perm, route ? &r : nullptr, n, m, x, g, dx, da, stream));
}

extern "C" laplex_status laplex_backward_phased(const float* a_sorted, const uint32_t* perm, const void* route, const float* phi,
                                                uint64_t n, uint32_t m, const float* x, const float* g, float* dx, float* da,
                                                float* dphi, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n == 0 || m == 0) return LAPLEX_OK;
  laplex_status st = check_apply_common(a_sorted, perm, n, m, x, dx, ws);
  if (st != LAPLEX_OK) return st;
  if (!phi || !g || !da || !dphi) return LAPLEX_ERR_NULL;
  if (misaligned(phi, 4) || misaligned(g, 4) || misaligned(da, 4) || misaligned(dphi, 4) || (route && misaligned(route, 256)))
    return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_backward(nullptr, n, 0, m, false, &need, true);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t xb = n * (size_t)m * 4, vb = n * 4, rb = route ? route_bytes(n) : 0;
  const void* outs[3] = {dx, da, dphi};
  const size_t outb[3] = {xb, vb, vb};
  for (int o = 0; o < 3; ++o) {
    const void* p = outs[o];
    const size_t pb = outb[o];
    if (overlaps(p, pb, x, xb) || overlaps(p, pb, g, xb) || overlaps(p, pb, phi, vb) || overlaps(p, pb, a_sorted, vb) ||
        overlaps(p, pb, perm, vb) || overlaps(p, pb, ws, ws_bytes) || overlaps(p, pb, route, rb))
      return LAPLEX_ERR_OVERLAP;
    for (int q = o + 1; q < 3; ++q)
      if (overlaps(p, pb, outs[q], outb[q])) return LAPLEX_ERR_OVERLAP;
  }
  const BackwardWorkspace bw = carve_backward(ws, n, 0, m, false, nullptr, true);
  SortRoute r{};
  if (route) r = carve_route(route, n);
  return from_hip(backward_phased(bw, a_sorted, perm, route ? &r : nullptr, phi, n, m, x, g, dx, da, dphi, stream));
}

extern "C" laplex_status laplex_backward_phased_general(const float* a_sorted, const uint32_t* perm_a, const void* route_a,
                                                        const float* phi, uint64_t n, const float* b_sorted,
                                                        const uint32_t* perm_b, const void* route_b, const float* psi,
                                                        uint64_t k, uint32_t m, const float* x, const float* g, float* dx,
                                                        float* da, float* db, float* dphi, float* dpsi, void* ws,
                                                        size_t ws_bytes, hipStream_t stream) {
  if (m == 0 || (n == 0 && k == 0)) return LAPLEX_OK;
  if (n > kMaxLen || k > kMaxLen || m > kMaxCols) return LAPLEX_ERR_SIZE;
  const size_t xb = k * (size_t)m * 4, gb = n * (size_t)m * 4, nb = n * 4, kb = k * 4;
  if (n == 0 || k == 0) {
    // no pairs: every gradient is zero (dx, db, dpsi when n == 0; da, dphi when k == 0)
    if (n == 0) {
      if (!dx || !db || !dpsi) return LAPLEX_ERR_NULL;
      if (misaligned(dx, 4) || misaligned(db, 4) || misaligned(dpsi, 4)) return LAPLEX_ERR_ALIGN;
      if (overlaps(dx, xb, db, kb) || overlaps(dx, xb, dpsi, kb) || overlaps(db, kb, dpsi, kb)) return LAPLEX_ERR_OVERLAP;
      hipError_t e = fill_zero_u32(dx, k * (uint64_t)m, stream);
      if (e == hipSuccess) e = fill_zero_u32(db, k, stream);
      if (e == hipSuccess) e = fill_zero_u32(dpsi, k, stream);
      return from_hip(e);
    }
    if (!da || !dphi) return LAPLEX_ERR_NULL;
    if (misaligned(da, 4) || misaligned(dphi, 4)) return LAPLEX_ERR_ALIGN;
    if (overlaps(da, nb, dphi, nb)) return LAPLEX_ERR_OVERLAP;
    hipError_t e = fill_zero_u32(da, n, stream);
    if (e == hipSuccess) e = fill_zero_u32(dphi, n, stream);
    return from_hip(e);
  }
  if (!a_sorted || !perm_a || !phi || !b_sorted || !perm_b || !psi || !x || !g || !dx || !da || !db || !dphi || !dpsi || !ws)
    return LAPLEX_ERR_NULL;
  const void* ins4[] = {a_sorted, perm_a, phi, b_sorted, perm_b, psi, x, g, dx, da, db, dphi, dpsi};
  for (const void* p : ins4)
    if (misaligned(p, 4)) return LAPLEX_ERR_ALIGN;
  if (misaligned(ws, 256) || (route_a && misaligned(route_a, 256)) || (route_b && misaligned(route_b, 256)))
    return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_backward(nullptr, n, k, m, true, &need, true);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t rab = route_a ? route_bytes(n) : 0, rbb = route_b ? route_bytes(k) : 0;
  const void* outs[5] = {dx, da, db, dphi, dpsi};
  const size_t outb[5] = {xb, nb, kb, nb, kb};
  for (int o = 0; o < 5; ++o) {
    const void* p = outs[o];
    const size_t pb = outb[o];
    if (overlaps(p, pb, x, xb) || overlaps(p, pb, g, gb) || overlaps(p, pb, a_sorted, nb) || overlaps(p, pb, perm_a, nb) ||
        overlaps(p, pb, phi, nb) || overlaps(p, pb, b_sorted, kb) || overlaps(p, pb, perm_b, kb) || overlaps(p, pb, psi, kb) ||
        overlaps(p, pb, ws, ws_bytes) || overlaps(p, pb, route_a, rab) || overlaps(p, pb, route_b, rbb))
      return LAPLEX_ERR_OVERLAP;
    for (int q = o + 1; q < 5; ++q)
      if (overlaps(p, pb, outs[q], outb[q])) return LAPLEX_ERR_OVERLAP;
  }
  const BackwardWorkspace bw = carve_backward(ws, n, k, m, true, nullptr, true);
  SortRoute ra{}, rb{};
  if (route_a) ra = carve_route(route_a, n);
  if (route_b) rb = carve_route(route_b, k);
  return from_hip(backward_phased_general(bw, a_sorted, perm_a, route_a ? &ra : nullptr, phi, n, b_sorted, perm_b,
                                          route_b ? &rb : nullptr, psi, k, m, x, g, dx, da, db, dphi, dpsi, stream));
}

extern "C" laplex_status laplex_backward_general(const float* a_sorted, const uint32_t* perm_a, const void* route_a, uint64_t n,
                                                 const float* b_sorted, const uint32_t* perm_b, const void* route_b, uint64_t k,
                                                 uint32_t m, const float* x, const float* g, float* dx, float* da, float* db,
                                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (m == 0 || (n == 0 && k == 0)) return LAPLEX_OK;
  if (n > kMaxLen || k > kMaxLen || m > kMaxCols) return LAPLEX_ERR_SIZE;
  const size_t xb = k * (size_t)m * 4, gb = n * (size_t)m * 4, nb = n * 4, kb = k * 4;
  if (n == 0 || k == 0) {
    // no pairs: every gradient is zero (dx and db when n == 0, da when k == 0)
    if (n == 0) {
      if (!dx || !db) return LAPLEX_ERR_NULL;
      if (misaligned(dx, 4) || misaligned(db, 4)) return LAPLEX_ERR_ALIGN;
      if (overlaps(dx, xb, db, kb)) return LAPLEX_ERR_OVERLAP;
      hipError_t e = fill_zero_u32(dx, k * (uint64_t)m, stream);
      if (e == hipSuccess) e = fill_zero_u32(db, k, stream);
      return from_hip(e);
    }
    if (!da) return LAPLEX_ERR_NULL;
    if (misaligned(da, 4)) return LAPLEX_ERR_ALIGN;
    return from_hip(fill_zero_u32(da, n, stream));
  }
  if (!a_sorted || !perm_a || !b_sorted || !perm_b || !x || !g || !dx || !da || !db || !ws) return LAPLEX_ERR_NULL;
  if (misaligned(a_sorted, 4) || misaligned(perm_a, 4) || misaligned(b_sorted, 4) || misaligned(perm_b, 4) ||
      misaligned(x, 4) || misaligned(g, 4) || misaligned(dx, 4) || misaligned(da, 4) || misaligned(db, 4) ||
      misaligned(ws, 256) || (route_a && misaligned(route_a, 256)) || (route_b && misaligned(route_b, 256)))
    return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_backward(nullptr, n, k, m, true, &need);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t rab = route_a ? route_bytes(n) : 0, rbb = route_b ? route_bytes(k) : 0;
  const void* outs[3] = {dx, da, db};
  const size_t outb[3] = {xb, nb, kb};
  for (int o = 0; o < 3; ++o) {
    const void* p = outs[o];
    const size_t pb = outb[o];
    if (overlaps(p, pb, x, xb) || overlaps(p, pb, g, gb) || overlaps(p, pb, a_sorted, nb) || overlaps(p, pb, perm_a, nb) ||
        overlaps(p, pb, b_sorted, kb) || overlaps(p, pb, perm_b, kb) || overlaps(p, pb, ws, ws_bytes) ||
        overlaps(p, pb, route_a, rab) || overlaps(p, pb, route_b, rbb))
      return LAPLEX_ERR_OVERLAP;
    for (int q = o + 1; q < 3; ++q)
      if (overlaps(p, pb, outs[q], outb[q])) return LAPLEX_ERR_OVERLAP;
  }
  const BackwardWorkspace bw = carve_backward(ws, n, k, m, true, nullptr);
  SortRoute ra{}, rb{};
  if (route_a) ra = carve_route(route_a, n);
  if (route_b) rb = carve_route(route_b, k);
  return from_hip(backward_general(bw, a_sorted, perm_a, route_a ? &ra : nullptr, n, b_sorted, perm_b, route_b ? &rb : nullptr,
                                   k, m, x, g, dx, da, db, stream));
}

extern "C" laplex_status laplex_gram_weighted(const float* a_sorted, const uint32_t* perm_a, uint64_t n, const float* b_sorted,
                                              const uint32_t* perm_b, uint64_t k, const float* D, uint64_t row_begin,
                                              uint64_t row_count, float* M, uint64_t ldm, void* ws, size_t ws_bytes,
                                              hipStream_t stream) {
  if (n == 0 || row_count == 0) return LAPLEX_OK;
  if (n > kMaxLen || k > kMaxLen || n > kGramMaxLen) return LAPLEX_ERR_SIZE;
  if (row_begin > n || row_count > n - row_begin || ldm < n) return LAPLEX_ERR_ARG;
  // the extent of M in bytes, ((row_count - 1) ldm + n) 4, must not overflow
  if (row_count > 1 && ldm > (UINT64_MAX / 4 - n) / (row_count - 1)) return LAPLEX_ERR_SIZE;
  if (!a_sorted || !perm_a || !M || !ws) return LAPLEX_ERR_NULL;
  if (k > 0 && (!b_sorted || !perm_b || !D)) return LAPLEX_ERR_NULL;
  if (misaligned(a_sorted, 4) || misaligned(perm_a, 4) || misaligned(M, 4) || misaligned(ws, 256) ||
      (k > 0 && (misaligned(b_sorted, 4) || misaligned(perm_b, 4) || misaligned(D, 4))))
    return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_gram(nullptr, n, k, &need);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t mb = ((row_count - 1) * ldm + n) * 4, nb = n * 4, kb = k * 4;
  if (overlaps(M, mb, a_sorted, nb) || overlaps(M, mb, perm_a, nb) || overlaps(M, mb, b_sorted, kb) ||
      overlaps(M, mb, perm_b, kb) || overlaps(M, mb, D, kb) || overlaps(M, mb, ws, ws_bytes))
    return LAPLEX_ERR_OVERLAP;
  const GramWorkspace g = carve_gram(ws, n, k, nullptr);
  return from_hip(gram_weighted(g, a_sorted, perm_a, n, b_sorted, perm_b, k, D, row_begin, row_count, M, ldm, stream));
}

extern "C" laplex_status laplex_matvec_general(const float* a_sorted, const uint32_t* perm_a, const void* route_a, uint64_t n,
                                               const float* b_sorted, const uint32_t* perm_b, const void* route_b, uint64_t k,
                                               uint32_t m, const float* x, float* y, void* ws, size_t ws_bytes,
                                               hipStream_t stream) {
  if (n == 0 || m == 0) return LAPLEX_OK;
  laplex_status st = check_apply_common(a_sorted, perm_a, n, m, x ? x : (const float*)y, y, ws);
  if (st != LAPLEX_OK) return st;
  if (k > kMaxLen) return LAPLEX_ERR_SIZE;
  if ((route_a && misaligned(route_a, 256)) || (route_b && misaligned(route_b, 256))) return LAPLEX_ERR_ALIGN;
  const size_t yb = n * (size_t)m * 4;
  if (k == 0) {
    if (overlaps(y, yb, a_sorted, n * 4) || overlaps(y, yb, perm_a, n * 4)) return LAPLEX_ERR_OVERLAP;
    return from_hip(fill_zero_u32(y, n * (uint64_t)m, stream));
  }
  if (!b_sorted || !perm_b || !x) return LAPLEX_ERR_NULL;
  if (misaligned(b_sorted, 4) || misaligned(perm_b, 4)) return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_apply(nullptr, k, n, n + k, m, Variant::Sym, true, &need);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t xb = k * (size_t)m * 4;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, a_sorted, n * 4) || overlaps(y, yb, perm_a, n * 4) ||
      overlaps(y, yb, b_sorted, k * 4) || overlaps(y, yb, perm_b, k * 4) || overlaps(y, yb, ws, ws_bytes) ||
      overlaps(y, yb, route_a, route_a ? route_bytes(n) : 0) || overlaps(y, yb, route_b, route_b ? route_bytes(k) : 0))
    return LAPLEX_ERR_OVERLAP;
  const ApplyWorkspace w = carve_apply(ws, k, n, n + k, m, Variant::Sym, true, nullptr);
  SortRoute ra{}, rb{};
  if (route_a) ra = carve_route(route_a, n);
  if (route_b) rb = carve_route(route_b, k);
  return from_hip(apply_general(w, Variant::Sym, a_sorted, perm_a, route_a ? &ra : nullptr, nullptr, n, b_sorted, perm_b,
                                route_b ? &rb : nullptr, nullptr, k, m, x, y, stream));
}

extern "C" laplex_status laplex_matvec_phased(const float* a_sorted, const uint32_t* perm_a, const void* route_a, const float* phi,
                                              uint64_t n, const float* b_sorted, const uint32_t* perm_b, const void* route_b,
                                              const float* psi, uint64_t k, uint32_t m, const float* x, float* y, void* ws,
                                              size_t ws_bytes, hipStream_t stream) {
  if (n == 0 || m == 0) return LAPLEX_OK;
  laplex_status st = check_apply_common(a_sorted, perm_a, n, m, x ? x : (const float*)y, y, ws);
  if (st != LAPLEX_OK) return st;
  if (!phi) return LAPLEX_ERR_NULL;
  if (misaligned(phi, 4)) return LAPLEX_ERR_ALIGN;
  if ((route_a && misaligned(route_a, 256)) || (route_b && misaligned(route_b, 256))) return LAPLEX_ERR_ALIGN;
  const size_t yb = n * (size_t)m * 4;
  SortRoute ra{}, rb{};
  if (route_a) ra = carve_route(route_a, n);
  if (b_sorted == nullptr) {
    if (!x) return LAPLEX_ERR_NULL;
    size_t need = 0;
    carve_apply(nullptr, n, n, n, m, Variant::Phased, false, &need);
    if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
    if (overlaps(y, yb, x, yb) || overlaps(y, yb, a_sorted, n * 4) || overlaps(y, yb, perm_a, n * 4) ||
        overlaps(y, yb, phi, n * 4) || overlaps(y, yb, ws, ws_bytes) || overlaps(y, yb, route_a, route_a ? route_bytes(n) : 0))
      return LAPLEX_ERR_OVERLAP;
    const ApplyWorkspace w = carve_apply(ws, n, n, n, m, Variant::Phased, false, nullptr);
    return from_hip(apply_sym(w, Variant::Phased, a_sorted, perm_a, route_a ? &ra : nullptr, phi, n, m, x, y, stream));
  }
  if (k > kMaxLen) return LAPLEX_ERR_SIZE;
  if (k == 0) {
    if (overlaps(y, yb, a_sorted, n * 4) || overlaps(y, yb, perm_a, n * 4) || overlaps(y, yb, phi, n * 4))
      return LAPLEX_ERR_OVERLAP;
    return from_hip(fill_zero_u32(y, n * (uint64_t)m, stream));
  }
  if (!perm_b || !psi || !x) return LAPLEX_ERR_NULL;
  if (misaligned(b_sorted, 4) || misaligned(perm_b, 4) || misaligned(psi, 4)) return LAPLEX_ERR_ALIGN;
  size_t need = 0;
  carve_apply(nullptr, k, n, n + k, m, Variant::Phased, true, &need);
  if (ws_bytes < need) return LAPLEX_ERR_WORKSPACE;
  const size_t xb = k * (size_t)m * 4;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, a_sorted, n * 4) || overlaps(y, yb, perm_a, n * 4) ||
      overlaps(y, yb, phi, n * 4) || overlaps(y, yb, b_sorted, k * 4) || overlaps(y, yb, perm_b, k * 4) ||
      overlaps(y, yb, psi, k * 4) || overlaps(y, yb, ws, ws_bytes) || overlaps(y, yb, route_a, route_a ? route_bytes(n) : 0) ||
      overlaps(y, yb, route_b, route_b ? route_bytes(k) : 0))
    return LAPLEX_ERR_OVERLAP;
  if (route_b) rb = carve_route(route_b, k);
  const ApplyWorkspace w = carve_apply(ws, k, n, n + k, m, Variant::Phased, true, nullptr);
  return from_hip(apply_general(w, Variant::Phased, a_sorted, perm_a, route_a ? &ra : nullptr, phi, n, b_sorted, perm_b,
                                route_b ? &rb : nullptr, psi, k, m, x, y, stream));
}

extern "C" const char* laplex_status_string(laplex_status s) {
  switch (s) {
    case LAPLEX_OK: return "ok";
    case LAPLEX_ERR_NULL: return "a required pointer is NULL";
    case LAPLEX_ERR_SIZE: return "size out of range (n, k < 2^32; m <= 65536)";
    case LAPLEX_ERR_ALIGN: return "misaligned pointer (arrays 4 bytes, workspace 256 bytes)";
    case LAPLEX_ERR_WORKSPACE: return "workspace too small";
    case LAPLEX_ERR_NONFINITE: return "an anchor is NaN or infinite";
    case LAPLEX_ERR_HIP: return "HIP runtime error";
    case LAPLEX_ERR_OVERLAP: return "an output overlaps an input or the workspace";
    case LAPLEX_ERR_STALLED: return "a look-back wait hit its spin limit";
    case LAPLEX_ERR_ARG: return "invalid argument";
    case LAPLEX_ERR_SCRATCH: return "call too large for the static scratch (LAPLEX_SCRATCH_BYTES)";
  }
  return "unknown status";
}

// ------------------------------------------------------------------ opt-in launch profiler
#include <atomic>
#include <mutex>
#include <vector>

namespace {
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<hipEvent_t> g_prof_ev;       // 2 per record: before, after
std::vector<const char*> g_prof_names;
std::vector<uint64_t> g_prof_units;
uint32_t g_prof_cap = 0, g_prof_cnt = 0;
}  // namespace

namespace laplex {
int prof_begin(hipStream_t s) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return -1;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_prof_cnt >= g_prof_cap) return -1;
  const int slot = (int)g_prof_cnt++;
  if (hipEventRecord(g_prof_ev[2 * slot], s) != hipSuccess) return -1;
  return slot;
}
void prof_end(int slot, const char* name, uint64_t units, hipStream_t s) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_names[slot] = name;
  g_prof_units[slot] = units;
  (void)hipEventRecord(g_prof_ev[2 * slot + 1], s);
}
}  // namespace laplex

extern "C" laplex_status laplex_profile_begin(uint32_t capacity) {
  if (capacity == 0 || capacity > (1u << 20)) return LAPLEX_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  while (g_prof_ev.size() < 2 * (size_t)capacity) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return LAPLEX_ERR_HIP;
    g_prof_ev.push_back(e);
  }
  g_prof_names.assign(capacity, nullptr);
  g_prof_units.assign(capacity, 0);
  g_prof_cap = capacity;
  g_prof_cnt = 0;
  g_prof_on.store(true);
  return LAPLEX_OK;
}

extern "C" uint32_t laplex_profile_end(void) {
  g_prof_on.store(false);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  return g_prof_cnt;
}

extern "C" laplex_status laplex_profile_get(uint32_t i, const char** name, float* ms, uint64_t* units) {
  if (!name || !ms || !units) return LAPLEX_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (i >= g_prof_cnt) return LAPLEX_ERR_ARG;
  if (hipEventSynchronize(g_prof_ev[2 * i + 1]) != hipSuccess) return LAPLEX_ERR_HIP;
  if (hipEventElapsedTime(ms, g_prof_ev[2 * i], g_prof_ev[2 * i + 1]) != hipSuccess) return LAPLEX_ERR_HIP;
  *name = g_prof_names[i];
  *units = g_prof_units[i];
  return LAPLEX_OK;
}
