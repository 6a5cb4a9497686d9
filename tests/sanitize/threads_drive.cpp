// Host-only drive of the C ABI from eight threads at once, under ThreadSanitizer: plans of
// every l created, queried and destroyed concurrently (the difference-set search is
// shared by all of them), size queries, dry runs and error strings.  Built and run by
// tests/test_host_sanitizers.py; a reported race ends the run with a nonzero status.
#include <atomic>
#include <cstdio>
#include <thread>
#include <vector>

#include "../../include/cqsa.h"

int main() {
  std::atomic<int> created{0};
  std::vector<std::thread> pool;
  for (int t = 0; t < 8; ++t) {
    pool.emplace_back([t, &created]() {
      const int32_t ls[] = {1, 2, 3, 4, 5, 6, 8, 9, 10};
      for (int rep = 0; rep < 3; ++rep) {
        for (int i = 0; i < 9; ++i) {
          const int32_t l = ls[(i + t) % 9];
          const int64_t c = int64_t(l) * (l - 1) + 1;
          cqsa_plan* p = nullptr;
          const uint32_t flags = (t & 1) ? CQSA_FLAG_CAUSAL : 0u;
          if (cqsa_plan_create(c * (3 + t), 2, 64, CQSA_BF16, &l, 1, 0, flags, &p) != CQSA_OK) {
            (void)cqsa_last_error();
            continue;
          }
          ++created;
          int64_t need = 0;
          (void)cqsa_plan_schedule(p, nullptr, 0, &need);
          std::vector<int64_t> s(need > 0 ? need : 1);
          (void)cqsa_plan_schedule(p, s.data(), need, &need);
          (void)cqsa_plan_coverage(p, nullptr, 0, &need);
          std::vector<int32_t> cov(need > 0 ? need : 1);
          (void)cqsa_plan_coverage(p, cov.data(), need, &need);
          cqsa_plan_info info;
          (void)cqsa_plan_info_get(p, &info);
          int64_t ws = 0;
          (void)cqsa_workspace_size(p, CQSA_RES_HOST_PINNED, &ws);
          cqsa_plan_destroy(p);
          int32_t ds[16];
          (void)cqsa_difference_set(l, ds, 16);
          (void)cqsa_difference_set(7, ds, 16);
          (void)cqsa_status_string(CQSA_EBUDGET);
        }
        const cqsa_rates r{1000.0, 5000.0, 50.0, 50.0};
        cqsa_estimate e;
        const int32_t l3[] = {3};
        // dry runs whose budget test the plan's shape settles (no tables built)
        (void)cqsa_plan_estimate(int64_t(1) << 22, 1, 128, CQSA_BF16, l3, 0, int64_t(1) << 31, CQSA_FLAG_PAD, &r, &e);
        (void)cqsa_plan_estimate(int64_t(1) << 30, 1, 128, CQSA_BF16, l3, 0, int64_t(1) << 31, CQSA_FLAG_PAD, &r, &e);
      }
    });
  }
  for (auto& th : pool) th.join();
  // a plan large enough that its tasks are built on several host threads, twice at once
  std::thread big[2];
  for (auto& th : big)
    th = std::thread([&created]() {
      const int32_t l4[] = {3, 3, 3, 3};
      cqsa_plan* p = nullptr;
      if (cqsa_plan_create(2401, 1, 64, CQSA_BF16, l4, 4, 0, 0, &p) == CQSA_OK) {
        ++created;
        cqsa_plan_destroy(p);
      }
    });
  for (auto& th : big) th.join();
  std::printf("plans created %d\n", created.load());
  return 0;
}
