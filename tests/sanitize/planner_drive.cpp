// Host-only drive of the planner under AddressSanitizer and UndefinedBehaviorSanitizer:
// plans, fallbacks and dry runs over many shapes, flags and budgets.  Built and run by
// tests/test_host_sanitizers.py; a sanitizer report ends the run with a nonzero status.
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../../memory_bounded_streaming_amd/csrc/plan.hpp"

using namespace cqsa;

// A causal plan's dispatch order must name every workgroup of the device-resident launch
// exactly once (entries decode to an item, head and tile the kernel indexes with), with -1
// only as padding; a plan without causality must have none.
static bool dispatch_ok(const Plan& p) {
  const bool causal = (p.flags & 0x8u) != 0;
  if (!causal || p.dev_order.empty()) return !(!causal && !p.dev_order.empty());
  const int64_t qt = p.dtype == CQSA_BF16 ? kAttnQueryTileBf16 : kAttnQueryTileF32;
  const int64_t tiles = (p.unit + qt - 1) / qt;
  const int64_t wgs = int64_t(p.dev_items.size()) * p.heads * tiles;
  if (p.dev_order.size() % 8 != 0) return false;
  std::vector<char> seen(wgs, 0);
  int64_t named = 0;
  for (int32_t v : p.dev_order) {
    if (v == -1) continue;
    if (v < 0 || v >= wgs || seen[v]) return false;
    seen[v] = 1;
    ++named;
  }
  return named == wgs;
}

int main() {
  int built = 0, refused = 0, bad_dispatch = 0;
  const std::vector<std::vector<int32_t>> level_sets = {{1}, {3}, {5}, {8}, {10}, {2, 2}, {3, 3}, {4, 2}, {3, 2, 2}};
  for (const auto& ls : level_sets) {
    int64_t prod_c = 1;
    for (int l : ls) prod_c *= l * (l - 1) + 1;
    for (int64_t n : {prod_c, prod_c * 7 + 1, prod_c * 16 - 3}) {
      for (uint32_t flags : {0u, 0x4u, 0xCu, 0x1u | 0x4u, 0x2u | 0x4u | 0x8u}) {
        for (int64_t budget : {int64_t(0), int64_t(1) << 20, int64_t(1) << 30}) {
          Plan p;
          std::string why;
          if (build_plan(n, 2, 64, CQSA_BF16, ls.data(), int(ls.size()), budget, flags, p, why) == CQSA_OK) {
            ++built;
            (void)descriptor_bytes(p);
            if (!dispatch_ok(p)) {
              ++bad_dispatch;
              std::printf("bad dispatch order: n %lld levels %zu flags 0x%x\n", (long long)n, ls.size(), flags);
            }
            if (budget > 0) {
              Plan f;
              std::string w;
              (void)fallback_plan(p, budget / 2, f, w);
            }
          } else {
            ++refused;
          }
          const cqsa_rates r{1.0, 1.0, 1.0, 1.0};
          cqsa_estimate e{};
          std::string w;
          (void)estimate_plan(n, 2, 64, CQSA_BF16, ls.data(), int(ls.size()), budget, flags, r, e, w);
        }
      }
    }
  }
  // automatic depth for very long inputs (estimated, not built)
  for (int64_t n : {int64_t(1) << 30, int64_t(12845056), int64_t(1376256)}) {
    const int32_t l3[] = {3};
    const cqsa_rates r{1000.0, 5000.0, 50.0, 50.0};
    cqsa_estimate e{};
    std::string w;
    (void)estimate_plan(n, 1, 128, CQSA_BF16, l3, 0, int64_t(2) << 30, 0x4u, r, e, w);
  }
  // causal plans with several heads and both dtypes, on the device-resident shape
  for (int heads : {1, 4, 8}) {
    for (cqsa_dtype dt : {CQSA_BF16, CQSA_F32}) {
      const int32_t l3[] = {3};
      Plan p;
      std::string why;
      if (build_plan(7 * 8192 + (heads == 4 ? 5 : 0), heads, 128, dt, l3, 1, 0, 0x8u | 0x4u, p, why) == CQSA_OK) {
        ++built;
        if (!dispatch_ok(p) || p.dev_order.empty()) {
          ++bad_dispatch;
          std::printf("bad dispatch order: heads %d dtype %d\n", heads, int(dt));
        }
      }
    }
  }
  std::printf("plans built %d, refused %d, bad dispatch orders %d\n", built, refused, bad_dispatch);
  return bad_dispatch != 0;
}
