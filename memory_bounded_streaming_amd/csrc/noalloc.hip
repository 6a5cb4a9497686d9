// Device-resident forward that allocates nothing: the partial slots and the forward
// descriptor tables live in one fixed array of device memory that the library holds on
// every device it runs on, instead of a workspace the caller passes or the library
// allocates.  For callers that cannot allocate (graph capture, tight serving loops).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "engine.hpp"
#include "plan.hpp"

namespace cqsa {

// Upper bound of the array: the partial slots (visits x N x H x (d + 2) float32, each of
// the two parts 256-byte aligned) plus the descriptor tables.
constexpr int64_t kStaticScratchBytes = int64_t(256) << 20;

}  // namespace cqsa

// One copy per device, loaded with this file's code object and held until the process
// ends.  Host code never uses this name as an address (on the host it is a stand-in);
// it uses the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[cqsa::kStaticScratchBytes];

namespace cqsa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the array on the current device, looked up once per device.
cqsa_status scratch_address(void*& out, std::string& why) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    why = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return CQSA_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    why = "device ordinal " + std::to_string(dev) + " is beyond the " + std::to_string(kMaxDevices) +
          " devices the static scratch supports";
    return CQSA_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      why = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return CQSA_EHIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  out = g_scratch_ptr[dev];
  return CQSA_OK;
}

}  // namespace

int64_t static_scratch_capacity() { return kStaticScratchBytes; }

int64_t static_scratch_need(const Plan& p) {
  return align_up(p.visits * p.n * p.heads * int64_t(p.d) * 4) + align_up(p.visits * p.n * p.heads * int64_t(2) * 4) +
         align_up(int64_t(p.dev_items.size()) * sizeof(WorkItem)) + align_up(int64_t(p.dev_runs.size()) * sizeof(KeyRun)) +
         align_up(int64_t(p.dev_order.size()) * int64_t(sizeof(int32_t)));
}

cqsa_status forward_static(const Plan& p, const void* q, const void* k, const void* v, void* o, float* lse,
                           hipStream_t stream, std::string& why) {
  const int64_t need = static_scratch_need(p);
  if (need > kStaticScratchBytes) {
    why = "the plan needs " + std::to_string(need) + " bytes of partial slots and descriptor tables; the static " +
          "scratch holds " + std::to_string(kStaticScratchBytes);
    return CQSA_ESMALL;
  }
  void* base = nullptr;
  cqsa_status st = scratch_address(base, why);
  if (st != CQSA_OK) return st;
  // layout: n slots | (m, l) slots | work items | key runs | dispatch order
  char* b = static_cast<char*>(base);
  const int64_t n_bytes = align_up(p.visits * p.n * p.heads * int64_t(p.d) * 4);
  const int64_t ml_bytes = align_up(p.visits * p.n * p.heads * int64_t(2) * 4);
  const int64_t it_bytes = align_up(int64_t(p.dev_items.size()) * sizeof(WorkItem));
  const int64_t run_bytes = align_up(int64_t(p.dev_runs.size()) * sizeof(KeyRun));
  float* n_slots = reinterpret_cast<float*>(b);
  float* ml_slots = reinterpret_cast<float*>(b + n_bytes);
  WorkItem* items = reinterpret_cast<WorkItem*>(b + n_bytes + ml_bytes);
  KeyRun* runs = reinterpret_cast<KeyRun*>(b + n_bytes + ml_bytes + it_bytes);
  int32_t* order = p.dev_order.empty() ? nullptr : reinterpret_cast<int32_t*>(b + n_bytes + ml_bytes + it_bytes + run_bytes);
  // The tables are rewritten on every call, in stream order: a call on another stream that
  // still runs reads the same array (calls that overlap on one device race).
  hipError_t e = hipMemcpyAsync(items, p.dev_items.data(), p.dev_items.size() * sizeof(WorkItem),
                                hipMemcpyHostToDevice, stream);
  if (e == hipSuccess && !p.dev_runs.empty())
    e = hipMemcpyAsync(runs, p.dev_runs.data(), p.dev_runs.size() * sizeof(KeyRun), hipMemcpyHostToDevice, stream);
  if (e == hipSuccess && order != nullptr)
    e = hipMemcpyAsync(order, p.dev_order.data(), p.dev_order.size() * sizeof(int32_t), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) {
    why = std::string("hipMemcpyAsync(descriptor tables): ") + hipGetErrorString(e);
    return CQSA_EHIP;
  }
  // Every visit slot of every row is written by the partial kernel before the merge
  // reads it, so nothing left in the array by an earlier call is read.
  st = run_partials_with(p, q, k, v, n_slots, ml_slots, items, runs, order, stream, why);
  if (st != CQSA_OK) return st;
  return run_merge(p, n_slots, ml_slots, o, lse, stream, why);
}

}  // namespace cqsa
