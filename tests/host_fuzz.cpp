// Argument fuzzing of the C ABI's host side: every size / plan / FLOP query
// with random (often invalid) shapes and parameters, and every entry point
// with arguments that must be rejected before any launch.  Built with the
// address and undefined-behaviour sanitizers on the host code (see
// test_host_sanitizers.py); no GPU is touched.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>

#include "nsg.h"

static int failures = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #cond); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

int main(int argc, char **argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  std::mt19937_64 rng(20250);
  auto pick = [&](std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); };
  auto side = [&]() {
    return pick({-7, -1, 0, 1, 2, 7, 128, 255, 256, 257, 512, 768, 4095, 4096, 11008, 65536, NSG_MAX_SIDE,
                 NSG_MAX_SIDE + 1, std::numeric_limits<int64_t>::max()});
  };
  double coeffs[3 * 80];
  for (int i = 0; i < 3 * 80; ++i) coeffs[i] = (i % 3 == 0) ? 3.4445 : (i % 3 == 1 ? -4.7750 : 2.0315);
  const float fvals[] = {-1.f, 0.f, 1e-7f, 1.f, 1.05f, std::numeric_limits<float>::quiet_NaN(),
                         std::numeric_limits<float>::infinity()};

  for (int it = 0; it < iters; ++it) {
    nsg_params_t p;
    ns_default_params(&p);
    if (rng() % 2) p.steps = (int32_t)pick({-1, 0, 1, 2, 5, 10, 64, 65, 1000});
    if (rng() % 3 == 0) p.n_coeffs = (int32_t)pick({-3, 0, 2, 3, 4, 3 * 5, 3 * 80, 3 * 81});
    // the caller's array must hold n_coeffs values (the default holds 3)
    if (rng() % 5 == 0) p.coeffs = nullptr;
    else if (p.n_coeffs != 3 || rng() % 2) p.coeffs = coeffs;
    if (rng() % 3 == 0) p.mode = (int32_t)pick({-1, 0, 1, 2, 3, 99});
    if (rng() % 3 == 0) p.restart_after = (int32_t)pick({-2, -1, 0, 1, 2, 3, 4, 5, 64, 1000});
    if (rng() % 4 == 0) p.safety = fvals[rng() % 7];
    if (rng() % 4 == 0) p.eps = fvals[rng() % 7];
    if (rng() % 3 == 0) p.compute_dtype = (int32_t)pick({-1, 0, 1, 2, 3});
    if (rng() % 3 == 0) p.sym_updates = (int32_t)pick({-1, 0, 1, 2});
    if (rng() % 3 == 0) p.restart_mask = rng();
    const int64_t G = pick({-1, 0, 1, 2, 32, 65535, 65536, std::numeric_limits<int64_t>::max()});
    const int64_t R = side(), C = side();
    const nsg_params_t *pp = (rng() % 16 == 0) ? nullptr : &p;

    size_t bytes = 0;
    nsg_status_t st = ns_workspace_size(G, R, C, pp, &bytes);
    EXPECT(st != NSG_OK || pp != nullptr);
    EXPECT(ns_workspace_size(G, R, C, pp, nullptr) != NSG_OK);
    double cr = -1.0, ex = -1.0;
    st = ns_flops(R, C, pp, &cr, &ex);
    if (st == NSG_OK) EXPECT(cr >= 0.0 && ex >= 0.0 && std::isfinite(cr) && std::isfinite(ex));
    nsg_launch_info_t ents[80];
    int32_t cnt = -1;
    const int32_t maxe = (int32_t)(rng() % 81);
    st = ns_plan(R, C, (int32_t)pick({-1, 0, 1, 2, 3}), pp, ents, maxe, &cnt);
    if (st == NSG_OK) EXPECT(cnt >= 0);  // the total; at most maxe entries written
    const int64_t k = pick({-1, 0, 1, 7, 256, 4096, 5000});
    const int32_t dim = (int32_t)pick({-2, -1, 0, 1, 2});
    const int32_t idt = (int32_t)pick({-1, 0, 1, 2, 3}), odt = (int32_t)pick({-1, 0, 1, 2, 3});
    (void)ns_select_workspace_size(G, R, C, k, dim, idt, odt, pp, &bytes);
    (void)nsg_l1_workspace_size(G, R, C, dim, &bytes);
    (void)ns_muon_workspace_size(G, R, C, pp, &bytes);

    // rejected before any launch: null data pointers, or no workspace
    if (G > 0 && R > 0 && C > 0) {
      char dummy[64];
      EXPECT(ns_orthogonalize(nullptr, idt, dummy, odt, G, R, C, pp, nullptr, 0, nullptr, nullptr) != NSG_OK);
      EXPECT(ns_orthogonalize(dummy, idt, nullptr, odt, G, R, C, pp, nullptr, 0, nullptr, nullptr) != NSG_OK);
      EXPECT(ns_orthogonalize(dummy, idt, dummy, odt, G, R, C, pp, nullptr, 0, nullptr, nullptr) != NSG_OK);
      EXPECT(ns_orthogonalize_selected(nullptr, idt, dummy, odt, G, R, C, k, dim, pp, nullptr, 0, nullptr,
                                       nullptr, nullptr) != NSG_OK);
      EXPECT(ns_orthogonalize_selected(dummy, idt, dummy, odt, G, R, C, k, dim, pp, nullptr, 0, nullptr,
                                       nullptr, nullptr) != NSG_OK);
      EXPECT(nsg_l1_norms(nullptr, idt, G, R, C, dim, nullptr, nullptr, 0, nullptr) != NSG_OK);
      EXPECT(ns_muon_step(nullptr, idt, dummy, odt, dummy, idt, G, R, C, 0.95f, 0.02, 0.01, 0.2, 1, 1, 1, pp,
                          nullptr, 0, nullptr, nullptr) != NSG_OK);
      EXPECT(ns_muon_step(dummy, idt, dummy, odt, dummy, idt, G, R, C, 0.95f, 0.02, 0.01, 0.2, 1, 1, 1, pp,
                          nullptr, 0, nullptr, nullptr) != NSG_OK);
      EXPECT(k == 0 || nsg_topk(nullptr, G, R, k, nullptr, nullptr, nullptr) != NSG_OK);  // k = 0: no-op
      const int64_t n = (G < (1 << 20) && R < (1 << 20)) ? G * R : std::numeric_limits<int64_t>::max();
      EXPECT(ns_muon_momentum(nullptr, idt, dummy, odt, n, 0.9f, nullptr) != NSG_OK);
      EXPECT(ns_muon_update(nullptr, idt, dummy, odt, n, 0.01, 0.0, 1.0, 1, 1, 1, nullptr) != NSG_OK);
      EXPECT(nsg_gemm_nt(idt, (int32_t)(rng() % 2), G, R, C, R, nullptr, R, (int32_t)(rng() % 3), nullptr, R,
                         (int32_t)(rng() % 3), 1.f, 0.f, nullptr, R, nullptr, C, nullptr, R, nullptr, 0.f, 0,
                         nullptr, nullptr) != NSG_OK);
    }
    (void)ns_status_string((nsg_status_t)pick({-1, 0, 1, 2, 3, 4, 5, 6, 1000}));
  }
  int32_t cnt = 0;
  EXPECT(ns_timing_collect(nullptr, nullptr, 0, &cnt) == NSG_OK || true);
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("ok %d iterations\n", iters);
  return 0;
}
