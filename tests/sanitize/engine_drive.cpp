// Host-sanitized drive of the stream engine on an MI355X: small plans in every staging
// mode, padded and causal, streamed forward and backward against the device path bit for
// bit.  The host code (planner, engine, C ABI, this drive) carries AddressSanitizer and
// UndefinedBehaviorSanitizer; the device code is built as usual.  Build (repository root):
//
//   mkdir -p _build/san
//   for f in abi plan engine; do
//     /opt/rocm/llvm/bin/clang++ -O1 -g -std=c++17 -fsanitize=address,undefined \
//       -fno-sanitize-recover=undefined -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include \
//       -c memory_bounded_streaming_amd/csrc/$f.cpp -o _build/san/$f.o; done
//   for f in kernels backward noalloc; do
//     hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
//       -c memory_bounded_streaming_amd/csrc/$f.hip -o _build/san/$f.o; done
//   hipcc --offload-arch=gfx950 -O1 -g -std=c++17 -Xarch_host -fsanitize=address \
//     -Xarch_host -fsanitize=undefined -c tests/sanitize/engine_drive.cpp -o _build/san/drive.o
//   hipcc --offload-arch=gfx950 -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
//     _build/san/*.o -o _build/san/engine_drive
//
// Run on the GPU with ASAN_OPTIONS=detect_leaks=0:halt_on_error=1; it prints one line per
// case and exits nonzero on a mismatch or a sanitizer report.  It leaves through _Exit so
// that the HIP runtime's own teardown does not run under the sanitizer's allocator.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>
#include "../../include/cqsa.h"

#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { std::printf("HIP %s at %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)
#define CQ(x) do { cqsa_status s_ = (x); if (s_ != CQSA_OK) { std::printf("cqsa %s (%s) at %d\n", cqsa_status_string(s_), cqsa_last_error(), __LINE__); return 1; } } while (0)

static uint64_t g_state = 88172645463325252ull;
static double urand() { g_state ^= g_state << 13; g_state ^= g_state >> 7; g_state ^= g_state << 17; return ((g_state >> 11) + 0.5) / 9007199254740992.0; }
static uint16_t bf16_of(float x) { uint32_t u; std::memcpy(&u, &x, 4); return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16); }

struct Case { std::vector<int32_t> ls; int64_t n; int h, d; uint32_t flags; };

int run(const Case& c) {
  const int64_t elems = c.n * c.h * c.d;
  const size_t bytes = size_t(elems) * 2;
  std::vector<uint16_t> host[4];
  for (auto& v : host) {
    v.resize(elems);
    for (auto& x : v) { double u1 = urand(), u2 = urand(); x = bf16_of(float(std::sqrt(-2 * std::log(u1)) * std::cos(6.283185307179586 * u2))); }
  }
  cqsa_plan* p = nullptr;
  CQ(cqsa_plan_create(c.n, c.h, c.d, CQSA_BF16, c.ls.data(), int32_t(c.ls.size()), 0, c.flags, &p));
  void* dv[9];
  for (auto& x : dv) CK(hipMalloc(&x, bytes));
  float* dl = nullptr;
  CK(hipMalloc(&dl, c.h * c.n * 4));
  for (int i = 0; i < 4; ++i) CK(hipMemcpy(dv[i], host[i].data(), bytes, hipMemcpyHostToDevice));
  // device path: forward (q,k,v -> o=dv[4], lse) then backward (dq, dk, dv = dv[5..7]); dO = dv[3]
  CQ(cqsa_forward(p, dv[0], dv[1], dv[2], dv[4], dl, CQSA_RES_DEVICE, nullptr, 0, nullptr, nullptr));
  CQ(cqsa_backward(p, dv[0], dv[1], dv[2], dv[4], dl, dv[3], dv[5], dv[6], dv[7], CQSA_RES_DEVICE, nullptr, 0, nullptr, nullptr));
  CK(hipDeviceSynchronize());
  std::vector<uint16_t> o_dev(elems), g_dev[3];
  std::vector<float> l_dev(c.h * c.n);
  CK(hipMemcpy(o_dev.data(), dv[4], bytes, hipMemcpyDeviceToHost));
  CK(hipMemcpy(l_dev.data(), dl, c.h * c.n * 4, hipMemcpyDeviceToHost));
  for (int i = 0; i < 3; ++i) { g_dev[i].resize(elems); CK(hipMemcpy(g_dev[i].data(), dv[5 + i], bytes, hipMemcpyDeviceToHost)); }
  // host-pinned path
  void* hp[9];
  for (auto& x : hp) CK(hipHostMalloc(&x, bytes, 0));
  float* hl = nullptr;
  CK(hipHostMalloc((void**)&hl, c.h * c.n * 4, 0));
  for (int i = 0; i < 4; ++i) std::memcpy(hp[i], host[i].data(), bytes);
  cqsa_stats st;
  CQ(cqsa_forward(p, hp[0], hp[1], hp[2], hp[4], hl, CQSA_RES_HOST_PINNED, nullptr, 0, nullptr, &st));
  int bad = std::memcmp(hp[4], o_dev.data(), bytes) != 0 || std::memcmp(hl, l_dev.data(), c.h * c.n * 4) != 0;
  // the streamed backward takes the device forward's O and LSE
  std::memcpy(hp[4], o_dev.data(), bytes);
  std::memcpy(hl, l_dev.data(), c.h * c.n * 4);
  CQ(cqsa_backward(p, hp[0], hp[1], hp[2], hp[4], hl, hp[3], hp[5], hp[6], hp[7], CQSA_RES_HOST_PINNED, nullptr, 0, nullptr, nullptr));
  for (int i = 0; i < 3; ++i) bad |= (std::memcmp(hp[5 + i], g_dev[i].data(), bytes) != 0) << (i + 1);
  std::printf("  levels %zu first l %d n %lld h %d d %d flags 0x%x: %s (h2d %lld B, d2d %lld B)\n", c.ls.size(), c.ls[0],
              (long long)c.n, c.h, c.d, c.flags, bad ? "MISMATCH" : "equal", (long long)st.bytes_h2d, (long long)st.bytes_d2d);
  std::fflush(stdout);
  for (auto& x : dv) CK(hipFree(x));
  CK(hipFree(dl));
  for (auto& x : hp) CK(hipHostFree(x));
  CK(hipHostFree(hl));
  cqsa_plan_destroy(p);
  return bad;
}

int main() {
  const uint32_t modes[] = {0u, CQSA_FLAG_HOST_ACC, CQSA_FLAG_KV_SINGLE, CQSA_FLAG_HOST_ACC | CQSA_FLAG_KV_SINGLE};
  std::vector<Case> cases;
  for (uint32_t m : modes) {
    cases.push_back({{3}, 7 * 96, 2, 128, m});
    cases.push_back({{2, 2}, 9 * 40 + 5, 1, 64, m | CQSA_FLAG_PAD});
    cases.push_back({{4}, 13 * 64, 2, 128, m | CQSA_FLAG_CAUSAL});
    cases.push_back({{3, 2}, 21 * 24 + 7, 1, 128, m | CQSA_FLAG_CAUSAL | CQSA_FLAG_PAD});
    cases.push_back({{8}, 57 * 16, 1, 64, m});
  }
  int fails = 0;
  for (auto& c : cases) {
    std::printf("case\n"); std::fflush(stdout);
    const int r = run(c);
    if (r < 0 || r > 15) return 1;
    fails += r != 0;
  }
  std::printf("%zu cases, %d mismatched\n", cases.size(), fails);
  std::fflush(stdout);
  // leave without running the runtime's static teardown
  std::_Exit(fails != 0);
}
