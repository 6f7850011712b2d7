// The tile-carry scan (k_tile_carry, laplex_scan.hpp) run on the CPU by the
// SIMT emulation in simt.hpp, for any tile count: each of its load widths
// (1, 2, 4, 8 and 16 tiles per thread) is chosen as the library's host code
// chooses it.  Test infrastructure.
//
// Inputs: T tiles, M columns; tile t has anchors (first, last) nondecreasing
// over the tiles, with a share of equal anchors at tile boundaries so that
// the tie decay (columns from tie_from on) sees weights of 1.  The program
// prints, as key=value lines:
//   err_f, err_b   max over columns and tiles of |carry - reference| /
//                  (the same recurrence over |aggregates|), for the carries
//                  from the left (cf) and from the right (cb); the reference
//                  is the plain recurrence in float64
//   nonfinite      carries holding a non-finite value
// Usage: sim_tile_carry T M tie_from seed
#include "hip/hip_runtime.h"
#include "laplex_scan.hpp"

#include <cmath>
#include <random>
#include <string>
#include <vector>

using namespace laplex;

int main(int argc, char** argv) {
  if (argc < 5) {
    std::fprintf(stderr, "usage: sim_tile_carry T M tie_from seed\n");
    return 2;
  }
  const uint64_t T = std::stoull(argv[1]);
  const uint32_t M = (uint32_t)std::stoul(argv[2]);
  const uint32_t tie_from = (uint32_t)std::stoul(argv[3]);
  std::mt19937_64 rng(std::stoull(argv[4]));
  std::uniform_real_distribution<float> step(0.f, 2.f), val(-1.f, 1.f), coin(0.f, 1.f);
  std::vector<float2> tanch(T);
  float s = 0.f;
  for (uint64_t t = 0; t < T; ++t) {
    const float first = (t > 0 && coin(rng) < 0.2f) ? s : s + step(rng);  // a tie with the previous tile's last anchor
    const float last = coin(rng) < 0.1f ? first : first + step(rng);      // a one-anchor tile
    tanch[t] = make_float2(first, last);
    s = last;
  }
  std::vector<float> bf(T * M), bb(T * M), cf(T * M, NAN), cb(T * M, NAN);
  for (auto& v : bf) v = val(rng);
  for (auto& v : bb) v = val(rng);

  const uint64_t q = (T + kCarryBlock - 1) / kCarryBlock;
  const float* pbf = bf.data();
  const float* pbb = bb.data();
  const float2* pan = tanch.data();
  float* pcf = cf.data();
  float* pcb = cb.data();
  auto run = [&](auto kernel) { simt::launch(dim3(M), dim3(kCarryBlock), [&] { kernel(pbf, pbb, pan, T, M, tie_from, pcf, pcb); }); };
  if (q <= 1)
    run(k_tile_carry<1>);
  else if (q <= 2)
    run(k_tile_carry<2>);
  else if (q <= 4)
    run(k_tile_carry<4>);
  else if (q <= 8)
    run(k_tile_carry<8>);
  else if (q <= (uint64_t)kCarryMaxQ)
    run(k_tile_carry<kCarryMaxQ>);
  else {
    std::fprintf(stderr, "T beyond one level\n");
    return 2;
  }

  // reference: L_t = bf_t + w(last_{t-1} - last_t) L_{t-1}, cf_t = L_{t-1};
  //            R_t = bb_t + w(first_t - first_{t+1}) R_{t+1}, cb_t = R_{t+1};
  // w = exp for the kernel's decay, 1 at 0 and 0 elsewhere for the tie decay
  // (the decays are taken in float32, as the kernel takes them)
  double err_f = 0.0, err_b = 0.0;
  uint64_t nonfinite = 0;
  for (uint32_t c = 0; c < M; ++c) {
    const bool tie = c >= tie_from;
    auto w = [&](float d) -> double { return tie ? (d == 0.f ? 1.0 : 0.0) : (double)decay(d); };
    double L = 0.0, La = 0.0;
    for (uint64_t t = 0; t < T; ++t) {
      const double got = cf[t * M + c];
      if (!std::isfinite(got)) ++nonfinite;
      err_f = std::max(err_f, std::fabs(got - L) / std::max(La, 1e-30));
      const double wt = t > 0 ? w(tanch[t - 1].y - tanch[t].y) : 0.0;
      L = bf[t * M + c] + wt * L;
      La = std::fabs(bf[t * M + c]) + wt * La;
    }
    double R = 0.0, Ra = 0.0;
    for (uint64_t t = T; t-- > 0;) {
      const double got = cb[t * M + c];
      if (!std::isfinite(got)) ++nonfinite;
      err_b = std::max(err_b, std::fabs(got - R) / std::max(Ra, 1e-30));
      const double wt = t + 1 < T ? w(tanch[t].x - tanch[t + 1].x) : 0.0;
      R = bb[t * M + c] + wt * R;
      Ra = std::fabs(bb[t * M + c]) + wt * Ra;
    }
  }
  std::printf("err_f=%.3e\nerr_b=%.3e\nnonfinite=%llu\nq=%llu\n", err_f, err_b, (unsigned long long)nonfinite,
              (unsigned long long)q);
  return 0;
}
