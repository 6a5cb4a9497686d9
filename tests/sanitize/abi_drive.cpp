// Host-only drive of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer:
// planner calls, size queries, argument checks and error paths (no GPU call is reached).
// Built and run by tests/test_host_sanitizers.py.
#include <cstdio>
#include <cstring>
#include <vector>
#include "../../include/cqsa.h"
int main() {
  int32_t ds[16];
  for (int l = -1; l <= 12; ++l) (void)cqsa_difference_set(l, ds, l > 0 && l < 16 ? l : 4);
  (void)cqsa_difference_set(3, nullptr, 3);
  (void)cqsa_difference_set(5, ds, 2);
  const std::vector<std::vector<int32_t>> sets = {{1}, {3}, {4}, {5}, {6}, {8}, {10}, {2, 2}, {3, 3}, {3, 2, 2}};
  int ok = 0;
  for (auto& ls : sets) {
    int64_t prod_c = 1;
    for (int l : ls) prod_c *= l * (l - 1) + 1;
    for (int64_t n : {prod_c * 5, prod_c * 5 + 3, prod_c - 1, int64_t(0), int64_t(-7)}) {
      for (uint32_t flags : {0u, 0x4u, 0x8u, 0xCu, 0x100u}) {
        for (int d : {64, 128, 96}) {
          cqsa_plan* p = nullptr;
          cqsa_status st = cqsa_plan_create(n, 2, d, CQSA_BF16, ls.data(), int32_t(ls.size()), 0, flags, &p);
          if (st != CQSA_OK) { (void)cqsa_last_error(); continue; }
          ++ok;
          cqsa_plan_info info;
          (void)cqsa_plan_info_get(p, &info);
          (void)cqsa_plan_info_get(p, nullptr);
          int64_t need = 0;
          (void)cqsa_plan_schedule(p, nullptr, 0, &need);
          std::vector<int64_t> buf(need > 0 ? need : 1);
          (void)cqsa_plan_schedule(p, buf.data(), need, &need);
          if (need > 1) (void)cqsa_plan_schedule(p, buf.data(), need - 1, &need);
          (void)cqsa_plan_coverage(p, nullptr, 0, &need);
          std::vector<int32_t> cov(need > 0 ? need : 1);
          (void)cqsa_plan_coverage(p, cov.data(), need, &need);
          if (need > 1) (void)cqsa_plan_coverage(p, cov.data(), need - 1, &need);
          int64_t ws = 0;
          (void)cqsa_workspace_size(p, CQSA_RES_DEVICE, &ws);
          (void)cqsa_workspace_size(p, CQSA_RES_HOST_PINNED, &ws);
          (void)cqsa_workspace_size(p, (cqsa_residency)5, &ws);
          (void)cqsa_backward_workspace_size(p, CQSA_RES_DEVICE, &ws);
          (void)cqsa_backward_workspace_size(p, CQSA_RES_HOST_PINNED, &ws);
          cqsa_plan* f = nullptr;
          if (cqsa_plan_fallback(p, int64_t(1) << 28, &f) == CQSA_OK) cqsa_plan_destroy(f);
          (void)cqsa_plan_fallback(p, 0, &f);
          (void)cqsa_plan_fallback(p, int64_t(1) << 28, nullptr);
          cqsa_plan_destroy(p);
        }
      }
    }
  }
  cqsa_plan_destroy(nullptr);
  cqsa_rates r{1000.0, 5000.0, 50.0, 50.0};
  cqsa_estimate e;
  const int32_t l3[] = {3};
  (void)cqsa_plan_estimate(int64_t(1) << 30, 1, 128, CQSA_BF16, l3, 0, int64_t(2) << 30, CQSA_FLAG_PAD, &r, &e);
  (void)cqsa_plan_estimate(int64_t(1) << 30, 1, 128, CQSA_BF16, l3, 0, int64_t(2) << 30, CQSA_FLAG_PAD, nullptr, &e);
  (void)cqsa_plan_estimate(int64_t(1) << 30, 1, 128, CQSA_BF16, nullptr, 1, 0, 0, &r, &e);
  (void)cqsa_debug_fail_allocations(-1);
  (void)cqsa_debug_fail_allocations(2);
  (void)cqsa_debug_fail_allocations(0);
  for (int s = -9; s <= 1; ++s) (void)cqsa_status_string((cqsa_status)s);
  std::printf("plans created %d; version %s\n", ok, cqsa_version());
  return 0;
}
