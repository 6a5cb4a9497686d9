// Execution of a CQS plan on one GPU.
//
// Device-resident path: one launch of the partial kernel over every (task, query unit)
// of the plan, each writing its visit slot, then one merge launch folding the slots of
// every row in ascending task order.
//
// Host-pinned path (the stream engine): "Stream-CQSA: Breaking the Billion-Token
// Barrier on a Single GPU" (wispaper explainer), section "Implementation: From
// High-Level Logic to GPU Kernels": divide, move each task's queries, keys and values to
// the device, form the task's softmax sums, aggregate them (in host memory when the device
// cannot hold the accumulator).  Tasks run in ascending id.  For each task the K/V
// segments are gathered into a staging buffer on the K/V copy stream; query units are
// streamed through a two-slot ring (Q block, partial block, accumulator block, output
// block) on the unit copy stream, which also returns each unit's accumulator or output
// blocks once its kernels have finished; the caller's stream runs the partial kernel and
// the merge.  Events order every reuse of a staging buffer; the unit stream's own order,
// behind the host's wait for a block's kernels, orders every reuse of a ring slot.
#include "engine.hpp"

#include <algorithm>
#include <atomic>
#include <chrono>
#include <deque>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <memory>
#include <utility>
#include <vector>

#include "kernels.hpp"

namespace cqsa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) {                                                                \
      why = std::string(#expr) + ": " + hipGetErrorString(e_);                             \
      return e_ == hipErrorOutOfMemory ? CQSA_ENOMEM : CQSA_EHIP;                          \
    }                                                                                      \
  } while (0)

float scale_log2(const Plan& p) { return static_cast<float>(1.0 / std::sqrt(double(p.d))) * kLog2e; }

// Device allocations of the library go through here: a test can make the next few fail
// as if the device were out of memory (cqsa_debug_fail_allocations).
std::atomic<int> g_fail_allocs{0};

hipError_t dev_malloc(void** ptr, int64_t bytes) {
  int pending = g_fail_allocs.load();
  while (pending > 0)
    if (g_fail_allocs.compare_exchange_weak(pending, pending - 1)) {
      *ptr = nullptr;
      return hipErrorOutOfMemory;
    }
  return hipMalloc(ptr, static_cast<size_t>(bytes));
}

// Observed device memory of a call: free memory at entry, and its minimum over the polls.
struct MemWatch {
  size_t free0 = 0, min_free = 0;
  bool ok = false;
  void begin() {
    size_t f = 0, t = 0;
    if (hipMemGetInfo(&f, &t) == hipSuccess) {
      free0 = min_free = f;
      ok = true;
    } else {
      (void)hipGetLastError();
    }
  }
  void poll() {
    if (!ok) return;
    size_t f = 0, t = 0;
    if (hipMemGetInfo(&f, &t) == hipSuccess)
      min_free = std::min(min_free, f);
    else
      (void)hipGetLastError();
  }
  int64_t peak() const { return ok ? static_cast<int64_t>(free0 - min_free) : -1; }
};

bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v != nullptr && v[0] != '\0' && v[0] != '0';
}

// Timing of the phases: begin/end event pairs per interval, read after the final
// synchronisation.  A phase's time is the union of its intervals, each placed on one
// time line by its offset from a reference event recorded first on the caller's stream
// (every engine stream waits for the caller before its first step), so intervals of
// one phase on two streams at once count once.
struct PhaseTimer {
  bool on = false;
  hipEvent_t ref = nullptr;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> spans[4];  // h2d, attn, merge, d2h
  hipError_t start(hipStream_t s) {
    if (!on) return hipSuccess;
    hipError_t e = hipEventCreate(&ref);
    if (e != hipSuccess) return e;
    return hipEventRecord(ref, s);
  }
  hipError_t begin(int phase, hipStream_t s, hipEvent_t& ev) {
    ev = nullptr;
    if (!on) return hipSuccess;
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return e;
    spans[phase].push_back({ev, nullptr});
    return hipEventRecord(ev, s);
  }
  hipError_t end(int phase, hipStream_t s) {
    if (!on) return hipSuccess;
    hipEvent_t ev;
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return e;
    spans[phase].back().second = ev;
    return hipEventRecord(ev, s);
  }
  double total(int phase) const {
    std::vector<std::pair<double, double>> iv;
    for (auto& sp : spans[phase]) {
      float b = 0, e = 0;
      if (!sp.first || !sp.second) continue;
      if (ref) {
        if (hipEventElapsedTime(&b, ref, sp.first) != hipSuccess || hipEventElapsedTime(&e, ref, sp.second) != hipSuccess)
          continue;
      } else if (hipEventElapsedTime(&e, sp.first, sp.second) != hipSuccess) {
        continue;
      }
      iv.push_back({b, e});
    }
    if (ref == nullptr) {  // one stream: the intervals do not overlap
      double ms = 0;
      for (auto& x : iv) ms += x.second - x.first;
      return ms;
    }
    std::sort(iv.begin(), iv.end());
    double ms = 0, cb = 0, ce = -1;
    bool open = false;
    for (auto& x : iv) {
      if (open && x.first <= ce) {
        ce = std::max(ce, x.second);
        continue;
      }
      if (open) ms += ce - cb;
      cb = x.first;
      ce = x.second;
      open = true;
    }
    if (open) ms += ce - cb;
    return ms;
  }
  ~PhaseTimer() {
    if (ref) (void)hipEventDestroy(ref);
    for (auto& v : spans)
      for (auto& sp : v) {
        if (sp.first) (void)hipEventDestroy(sp.first);
        if (sp.second) (void)hipEventDestroy(sp.second);
      }
  }
};

enum { PH_H2D = 0, PH_ATTN = 1, PH_MERGE = 2, PH_D2H = 3 };

// The host-pinned paths copy with explicit host <-> device directions and overlap the
// copies with compute, so every host tensor must be pinned host memory (hipHostMalloc,
// torch pin_memory).  A device pointer or pageable memory is rejected before any copy.
cqsa_status check_pinned(std::initializer_list<std::pair<const void*, const char*>> ps, std::string& why) {
  for (const auto& pr : ps) {
    if (pr.first == nullptr) continue;
    hipPointerAttribute_t a{};
    const hipError_t e = hipPointerGetAttributes(&a, pr.first);
    if (e != hipSuccess) (void)hipGetLastError();  // pageable memory may be reported as an error
    if (e != hipSuccess || a.type != hipMemoryTypeHost) {
      why = std::string(pr.second) +
            " is not pinned host memory (the host-pinned residency needs hipHostMalloc or pin_memory buffers)";
      return CQSA_EINVAL;
    }
  }
  return CQSA_OK;
}

}  // namespace

// ----------------------------------------------------------------------------------
// descriptor tables
// ----------------------------------------------------------------------------------
cqsa_status device_tables(const Plan& p, DeviceTables& out, std::string& why) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  const int64_t b0 = align_up(int64_t(p.dev_items.size()) * sizeof(WorkItem));
  const int64_t b1 = align_up(int64_t(p.dev_runs.size()) * sizeof(KeyRun));
  const int64_t b2 = align_up(int64_t(p.stream_items.size()) * sizeof(WorkItem));
  const int64_t b3 = align_up(int64_t(p.stream_runs.size()) * sizeof(KeyRun));
  const int64_t b4 = align_up(int64_t(p.dev_kitems.size()) * sizeof(WorkItem));
  const int64_t b5 = align_up(int64_t(p.dev_kruns.size()) * sizeof(KeyRun));
  const int64_t b6 = align_up(int64_t(p.bstream_items.size()) * sizeof(WorkItem));
  const int64_t b7 = align_up(int64_t(p.bstream_kitems.size()) * sizeof(WorkItem));
  const int64_t b8 = align_up(int64_t(p.bstream_kruns.size()) * sizeof(KeyRun));
  const int64_t b9 = align_up(int64_t(p.dev_order.size()) * int64_t(sizeof(int32_t)));
  std::lock_guard<std::mutex> lock(p.dev_mu);
  char* base = nullptr;
  for (auto& e : p.dev_tables)
    if (e.first == dev) base = static_cast<char*>(e.second);
  if (base == nullptr) {
    std::vector<char> host(b0 + b1 + b2 + b3 + b4 + b5 + b6 + b7 + b8 + b9, 0);
    // tables a plan does not use are empty (their data() may be null, which memcpy may
    // not receive even for zero bytes)
    auto put = [&](int64_t at, const auto& v) {
      if (!v.empty()) std::memcpy(host.data() + at, v.data(), v.size() * sizeof(v[0]));
    };
    put(0, p.dev_items);
    put(b0, p.dev_runs);
    put(b0 + b1, p.stream_items);
    put(b0 + b1 + b2, p.stream_runs);
    put(b0 + b1 + b2 + b3, p.dev_kitems);
    put(b0 + b1 + b2 + b3 + b4, p.dev_kruns);
    put(b0 + b1 + b2 + b3 + b4 + b5, p.bstream_items);
    put(b0 + b1 + b2 + b3 + b4 + b5 + b6, p.bstream_kitems);
    put(b0 + b1 + b2 + b3 + b4 + b5 + b6 + b7, p.bstream_kruns);
    put(b0 + b1 + b2 + b3 + b4 + b5 + b6 + b7 + b8, p.dev_order);
    void* mem = nullptr;
    HIP_TRY(dev_malloc(&mem, static_cast<int64_t>(host.size())));
    hipError_t e = hipMemcpy(mem, host.data(), host.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(mem);
      why = std::string("hipMemcpy(descriptor tables): ") + hipGetErrorString(e);
      return CQSA_EHIP;
    }
    p.dev_tables.push_back({dev, mem});
    base = static_cast<char*>(mem);
  }
  out.dev_items = reinterpret_cast<const WorkItem*>(base);
  out.dev_runs = reinterpret_cast<const KeyRun*>(base + b0);
  out.stream_items = reinterpret_cast<const WorkItem*>(base + b0 + b1);
  out.stream_runs = reinterpret_cast<const KeyRun*>(base + b0 + b1 + b2);
  out.dev_kitems = reinterpret_cast<const WorkItem*>(base + b0 + b1 + b2 + b3);
  out.dev_kruns = reinterpret_cast<const KeyRun*>(base + b0 + b1 + b2 + b3 + b4);
  out.bstream_items = reinterpret_cast<const WorkItem*>(base + b0 + b1 + b2 + b3 + b4 + b5);
  out.bstream_kitems = reinterpret_cast<const WorkItem*>(base + b0 + b1 + b2 + b3 + b4 + b5 + b6);
  out.bstream_kruns = reinterpret_cast<const KeyRun*>(base + b0 + b1 + b2 + b3 + b4 + b5 + b6 + b7);
  out.dev_order = p.dev_order.empty() ? nullptr
                                      : reinterpret_cast<const int32_t*>(base + b0 + b1 + b2 + b3 + b4 + b5 + b6 + b7 + b8);
  out.dev_order_len = static_cast<int64_t>(p.dev_order.size());
  out.bytes = b0 + b1 + b2 + b3 + b4 + b5 + b6 + b7 + b8 + b9;
  return CQSA_OK;
}

int64_t table_bytes(const Plan& p) { return descriptor_bytes(p); }

void set_fail_allocations(int count) { g_fail_allocs.store(count); }

void free_host_cache(const Plan& p) {
  std::lock_guard<std::mutex> lock(p.host_mu);
  if (p.host_acc_cache) (void)hipHostFree(p.host_acc_cache);
  p.host_acc_cache = nullptr;
  p.host_acc_cache_bytes = 0;
  p.host_acc_busy = false;
}

void free_device_tables(const Plan& p) {
  std::lock_guard<std::mutex> lock(p.dev_mu);
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto& e : p.dev_tables) {
    if (have) (void)hipSetDevice(e.first);
    (void)hipFree(e.second);
  }
  if (have) (void)hipSetDevice(cur);
  p.dev_tables.clear();
}

// ----------------------------------------------------------------------------------
// device-resident path
// ----------------------------------------------------------------------------------
cqsa_status run_partials(const Plan& p, const void* q, const void* k, const void* v, float* n_out,
                         float* ml_out, hipStream_t stream, std::string& why) {
  DeviceTables t{};
  cqsa_status st = device_tables(p, t, why);
  if (st != CQSA_OK) return st;
  return run_partials_with(p, q, k, v, n_out, ml_out, t.dev_items, t.dev_runs, t.dev_order, stream, why);
}

cqsa_status run_partials_with(const Plan& p, const void* q, const void* k, const void* v, float* n_out,
                              float* ml_out, const WorkItem* items, const KeyRun* runs, const int32_t* order,
                              hipStream_t stream, std::string& why) {
  AttnLaunch a{};
  a.dtype = p.dtype;
  a.d = p.d;
  a.heads = p.heads;
  a.q = q;
  a.k = k;
  a.v = v;
  a.n_out = n_out;
  a.ml_out = ml_out;
  a.items = items;
  a.runs = runs;
  a.n_items = static_cast<int>(p.dev_items.size());
  a.q_len = static_cast<int>(p.unit);
  a.order = order;
  a.order_len = order != nullptr ? static_cast<int64_t>(p.dev_order.size()) : 0;
  a.scale_log2 = scale_log2(p);
  HIP_TRY(launch_attn(a, stream));
  return CQSA_OK;
}

cqsa_status run_merge(const Plan& p, const float* n_in, const float* ml_in, void* o, float* lse,
                      hipStream_t stream, std::string& why) {
  MergeLaunch m{};
  m.dtype = p.dtype;
  m.d = p.d;
  m.heads = p.heads;
  m.rows = p.n;
  m.n_a = n_in;
  m.ml_a = ml_in;
  m.b_stride_n = p.n * p.heads * int64_t(p.d);
  m.b_stride_ml = p.n * p.heads * int64_t(2);
  m.n_b = n_in + m.b_stride_n;
  m.ml_b = ml_in + m.b_stride_ml;
  m.nb = static_cast<int>(p.visits - 1);
  m.final_out = true;
  m.o_out = o;
  m.lse_out = lse;
  m.lse_stride = p.n;
  m.lse_row0 = 0;
  HIP_TRY(launch_merge(m, stream));
  return CQSA_OK;
}

namespace {

cqsa_status forward_device(const Plan& p, const void* q, const void* k, const void* v, void* o, float* lse,
                           void* ws, int64_t ws_bytes, hipStream_t stream, cqsa_stats* stats, std::string& why) {
  if (p.budget > 0 && p.device_ws + table_bytes(p) > p.budget) {
    why = "device-resident path needs " + std::to_string(p.device_ws) + " workspace bytes and " +
          std::to_string(table_bytes(p)) + " descriptor bytes, over the budget";
    return CQSA_EBUDGET;
  }
  MemWatch mw;
  if (stats) mw.begin();
  bool owned = false;
  if (ws == nullptr) {
    HIP_TRY(dev_malloc(&ws, p.device_ws));
    owned = true;
  } else if (ws_bytes < p.device_ws) {
    why = "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(p.device_ws);
    return CQSA_ESMALL;
  }
  float* n_slots = static_cast<float*>(ws);
  float* ml_slots = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(p.visits * p.n * p.heads * int64_t(p.d) * 4));
  PhaseTimer tm;
  tm.on = stats != nullptr;
  const auto t0 = std::chrono::steady_clock::now();
  hipEvent_t ev;
  cqsa_status st = CQSA_OK;
  auto fail = [&](cqsa_status s) {
    if (owned) {
      (void)hipStreamSynchronize(stream);
      (void)hipFree(ws);
    }
    return s;
  };
  if (tm.begin(PH_ATTN, stream, ev) != hipSuccess) return fail(CQSA_EHIP);
  st = run_partials(p, q, k, v, n_slots, ml_slots, stream, why);
  mw.poll();
  if (st != CQSA_OK) return fail(st);
  if (tm.end(PH_ATTN, stream) != hipSuccess || tm.begin(PH_MERGE, stream, ev) != hipSuccess) return fail(CQSA_EHIP);
  st = run_merge(p, n_slots, ml_slots, o, lse, stream, why);
  if (st != CQSA_OK) return fail(st);
  if (tm.end(PH_MERGE, stream) != hipSuccess) return fail(CQSA_EHIP);
  if (owned || stats) {
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
      why = std::string("hipStreamSynchronize: ") + hipGetErrorString(e);
      return fail(CQSA_EHIP);
    }
  }
  mw.poll();
  if (owned) (void)hipFree(ws);
  if (stats) {
    std::memset(stats, 0, sizeof(*stats));
    stats->t_total_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    stats->t_attn_ms = tm.total(PH_ATTN);
    stats->t_merge_ms = tm.total(PH_MERGE);
    stats->peak_device_bytes = p.device_ws + table_bytes(p);
    stats->n_attn_launches = 1;
    stats->n_merge_launches = 1;
    stats->useful_flop = p.useful_flop();
    stats->observed_peak_bytes = mw.peak();
    stats->device_free_at_entry = static_cast<int64_t>(mw.free0);
    stats->levels_used = static_cast<int32_t>(p.ls.size());
  }
  return CQSA_OK;
}

// How many tasks the host may enqueue ahead of the one the device is finishing.
#ifndef CQSA_TASKS_AHEAD
#define CQSA_TASKS_AHEAD 2
#endif
constexpr int kTasksAhead = CQSA_TASKS_AHEAD;

// RAII holder of the stream engine's HIP objects.
// The engine adds two streams (K/V staging copies; query-unit copies in and out) to the
// caller's stream, which runs the kernels.  Copies out share the stream of the copies in:
// on a stream of their own, behind a wait for another stream's event, the runtime ran
// them at a fraction of the link's rate or as copy kernels on the compute units.
struct StreamRes {
  hipStream_t s[2] = {nullptr, nullptr};  // kv, io
  hipStream_t caller = nullptr;
  std::vector<hipEvent_t> events;
  void* ws = nullptr;
  bool own_ws = false;
  float* host_acc = nullptr;
  const Plan* acc_plan = nullptr;  // host_acc is the plan's cached accumulator, lent for the call
  ~StreamRes() {
    (void)hipStreamSynchronize(caller);
    for (hipStream_t x : s)
      if (x) (void)hipStreamSynchronize(x);
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
    for (hipStream_t x : s)
      if (x) (void)hipStreamDestroy(x);
    if (own_ws && ws) (void)hipFree(ws);
    if (acc_plan) {
      std::lock_guard<std::mutex> lock(acc_plan->host_mu);
      acc_plan->host_acc_busy = false;
    } else if (host_acc) {
      (void)hipHostFree(host_acc);
    }
  }
  // The pinned host accumulator: the plan's cached one when it is free and large enough
  // (allocated on the first call), else one of this call's own.
  hipError_t lend_host_acc(const Plan& p, int64_t bytes) {
    {
      std::lock_guard<std::mutex> lock(p.host_mu);
      if (!p.host_acc_busy) {
        if (p.host_acc_cache == nullptr || p.host_acc_cache_bytes < bytes) {
          if (p.host_acc_cache) (void)hipHostFree(p.host_acc_cache);
          p.host_acc_cache = nullptr;
          p.host_acc_cache_bytes = 0;
          hipError_t e = hipHostMalloc(&p.host_acc_cache, static_cast<size_t>(bytes), hipHostMallocDefault);
          if (e != hipSuccess) return e;
          p.host_acc_cache_bytes = bytes;
        }
        p.host_acc_busy = true;
        acc_plan = &p;
        host_acc = static_cast<float*>(p.host_acc_cache);
        return hipSuccess;
      }
    }
    return hipHostMalloc(reinterpret_cast<void**>(&host_acc), static_cast<size_t>(bytes), hipHostMallocDefault);
  }
  hipError_t event(hipEvent_t& e) {
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r == hipSuccess) events.push_back(e);
    return r;
  }
};

// Guard words around the pieces of a workspace the library allocated (CQSA_CANARY=1):
// filled before the call, compared after it.
constexpr int64_t kGuardBytes = 256;
constexpr uint32_t kGuardWord = 0xC0DEC0DEu;

struct Canary {
  bool on = false;
  std::vector<std::pair<char*, std::string>> guards;  // guard address, piece name
  hipError_t fill(hipStream_t s) {
    for (auto& g : guards) {
      hipError_t e = hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(g.first), static_cast<int>(kGuardWord),
                                       kGuardBytes / 4, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // the name of the first piece whose guard changed, "" if none
  std::string check() const {
    std::vector<uint32_t> host(kGuardBytes / 4);
    for (auto& g : guards) {
      if (hipMemcpy(host.data(), g.first, kGuardBytes, hipMemcpyDeviceToHost) != hipSuccess) return g.second + " (unreadable)";
      for (uint32_t w : host)
        if (w != kGuardWord) return g.second;
    }
    return "";
  }
};

// One attempt of the streamed forward with plan p.  dev_oom reports that the device
// workspace (or the descriptor tables) could not be allocated, the failure the caller
// recovers from by re-planning.
cqsa_status forward_stream(const Plan& p, const char* q, const char* k, const char* v, char* o, float* lse,
                           void* ws, int64_t ws_bytes, hipStream_t caller, cqsa_stats* stats, MemWatch& mw,
                           bool& dev_oom, std::string& why) {
  dev_oom = false;
  const auto t0 = std::chrono::steady_clock::now();
  const Footprint fp = p.stream_fp;
  const StreamLayout L = stream_layout(p, fp.acc_on_device, fp.kv_buffers);
  const bool sync = env_on("CQSA_SYNC");
  Canary canary;
  canary.on = ws == nullptr && env_on("CQSA_CANARY");
  DeviceTables tabs{};
  cqsa_status st = device_tables(p, tabs, why);
  if (st == CQSA_ENOMEM) dev_oom = true;
  if (st != CQSA_OK) return st;
  mw.poll();

  StreamRes res;
  const int kPieces = 2 * fp.kv_buffers + 2 * 7 + 3;  // upper bound of the pieces carved below
  if (ws == nullptr) {
    const int64_t bytes = L.total + (canary.on ? kPieces * kGuardBytes : 0);
    const hipError_t e = dev_malloc(&res.ws, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      why = "device workspace of " + std::to_string(bytes) + " bytes: " + hipGetErrorString(e);
      dev_oom = e == hipErrorOutOfMemory;
      return dev_oom ? CQSA_ENOMEM : CQSA_EHIP;
    }
    res.own_ws = true;
  } else {
    if (ws_bytes < L.total) {
      why = "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(L.total);
      return CQSA_ESMALL;
    }
    res.ws = ws;
  }
  mw.poll();
  // carve the workspace (a guard follows every piece in canary mode)
  char* cur = static_cast<char*>(res.ws);
  auto take = [&](int64_t bytes, const char* name) {
    char* r = cur;
    cur += bytes;
    if (canary.on) {
      canary.guards.push_back({cur, name});
      cur += kGuardBytes;
    }
    return r;
  };
  char* kst[2] = {nullptr, nullptr};
  char* vst[2] = {nullptr, nullptr};
  for (int b = 0; b < fp.kv_buffers; ++b) {
    kst[b] = take(L.kv_stage, "K staging");
    vst[b] = take(L.kv_stage, "V staging");
  }
  struct Slot {
    char* q;
    float* n;
    float* ml;
    float* an;
    float* aml;
    char* o;
    float* lse;
  } slot[2];
  for (auto& s : slot) {
    s.q = take(L.q_blk, "Q block");
    s.n = reinterpret_cast<float*>(take(L.n_blk, "partial n block"));
    s.ml = reinterpret_cast<float*>(take(L.ml_blk, "partial (m, l) block"));
    s.an = fp.acc_on_device ? nullptr : reinterpret_cast<float*>(take(L.n_blk, "accumulator n block"));
    s.aml = fp.acc_on_device ? nullptr : reinterpret_cast<float*>(take(L.ml_blk, "accumulator (m, l) block"));
    s.o = take(L.o_blk, "O block");
    s.lse = L.lse_blk ? reinterpret_cast<float*>(take(L.lse_blk, "LSE block")) : nullptr;
  }
  float* lse_dev = L.lse_all ? reinterpret_cast<float*>(take(L.lse_all, "LSE")) : nullptr;
  float* acc_n = fp.acc_on_device ? reinterpret_cast<float*>(take(L.acc_n, "accumulator n")) : nullptr;
  float* acc_ml = fp.acc_on_device ? reinterpret_cast<float*>(take(L.acc_ml, "accumulator (m, l)")) : nullptr;

  const int64_t H = p.heads, D = p.d, U = p.unit, N = p.n;
  const int64_t row_in = p.row_in_bytes();
  const int64_t nrow_f = H * D;  // floats of n per token row
  const int64_t mlrow_f = H * 2;
  float* host_n = nullptr;
  float* host_ml = nullptr;
  if (!fp.acc_on_device) {
    HIP_TRY(res.lend_host_acc(p, N * (nrow_f + mlrow_f) * int64_t(sizeof(float))));
    host_n = res.host_acc;
    host_ml = res.host_acc + N * nrow_f;
  }
  res.caller = caller;
  for (auto& s : res.s) HIP_TRY(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
  mw.poll();
  // K/V staging copies on one stream; the query-unit copies in (Q and accumulator blocks)
  // and out (accumulator, O and LSE blocks) on another, in the order they are needed; the
  // kernels on the caller's stream
  hipStream_t s_kv = res.s[0], s_io = res.s[1], s_c = caller;
  hipEvent_t start, kv_ready[2], kv_free[2], q_ready[2], c_done[2], task_done[kTasksAhead + 1], all_merged;
  HIP_TRY(res.event(start));
  HIP_TRY(res.event(all_merged));
  for (int i = 0; i <= kTasksAhead; ++i) HIP_TRY(res.event(task_done[i]));
  for (int i = 0; i < 2; ++i) {
    HIP_TRY(res.event(kv_ready[i]));
    HIP_TRY(res.event(kv_free[i]));
    HIP_TRY(res.event(q_ready[i]));
    HIP_TRY(res.event(c_done[i]));
  }
  PhaseTimer tm;
  tm.on = stats != nullptr;
  HIP_TRY(tm.start(caller));
  if (canary.on) HIP_TRY(canary.fill(caller));
  HIP_TRY(hipEventRecord(start, caller));
  HIP_TRY(hipStreamWaitEvent(s_kv, start, 0));
  HIP_TRY(hipStreamWaitEvent(s_io, start, 0));
  auto step = [&]() -> hipError_t { return sync ? hipDeviceSynchronize() : hipSuccess; };

  hipEvent_t tev;
  int64_t bytes_h2d = 0, bytes_d2h = 0, bytes_d2d = 0, n_attn = 0, n_merge = 0, n_h2d = 0, n_d2h = 0;
  // Every host <-> device copy is timed on its own (the union of the copies' intervals is
  // the phase's busy time, as a copy trace counts it); device copies are not timed.
  auto copy = [&](int phase, void* dst, const void* src, int64_t bytes, hipMemcpyKind kind, hipStream_t s) {
    hipError_t e = phase >= 0 ? tm.begin(phase, s, tev) : hipSuccess;
    if (e == hipSuccess) e = hipMemcpyAsync(dst, src, static_cast<size_t>(bytes), kind, s);
    if (e == hipSuccess && phase >= 0) e = tm.end(phase, s);
    return e;
  };
  const int64_t tu = p.task_units;
  const float c2 = scale_log2(p);
  const int64_t e = p.elem_bytes();
  std::vector<int64_t> last_block(p.n_units, -4);  // ring block that last wrote a unit's host accumulator
  int64_t blk = 0;

  const bool progress = std::getenv("CQSA_PROGRESS") != nullptr;
  const int64_t n_tasks = static_cast<int64_t>(p.tasks.size());
  auto report = [&](int64_t done) {
    const double s = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    std::fprintf(stderr, "cqsa: task %lld/%lld done, %.1f s\n", static_cast<long long>(done + 1),
                 static_cast<long long>(n_tasks), s);
    std::fflush(stderr);
  };
  // Device-to-host copies are enqueued only once the kernels they wait for have finished,
  // on the stream that then carries the next inputs: a copy enqueued behind a wait on
  // another stream's event, long before that event completes, ran at a fraction of the
  // link's rate (12.8 against 56.8 GB/s, more often the further ahead the host ran).  The
  // host therefore stays two blocks ahead of the device: before block k's inputs it waits
  // for block k-2's kernels and enqueues that block's copies, which precede block k's
  // inputs into the same ring slot on the stream.
  struct PendingD2H {
    int64_t blk;
    int j;
    int64_t pu, R;
    bool first, last;
  };
  std::deque<PendingD2H> pending;
  auto flush_d2h = [&](int64_t upto) -> hipError_t {
    while (!pending.empty() && pending.front().blk <= upto) {
      const PendingD2H r = pending.front();
      pending.pop_front();
      const Slot& S = slot[r.j];
      // the host has seen the block's kernels finish, so the copies need no wait on the device
      hipError_t err = hipEventSynchronize(c_done[r.j]);
      if (err != hipSuccess) return err;
      if (r.last) {
        err = copy(PH_D2H, o + r.pu * U * H * D * e, S.o, r.R * H * D * e, hipMemcpyDeviceToHost, s_io);
        if (err != hipSuccess) return err;
        bytes_d2h += r.R * H * D * e;
        ++n_d2h;
        if (lse != nullptr && lse_dev == nullptr) {
          // LSE is [H][N] on the host and [H][U] in the block: one contiguous copy per head
          for (int64_t hh = 0; hh < H && err == hipSuccess; ++hh)
            err = copy(PH_D2H, lse + hh * N + r.pu * U, S.lse + hh * U, r.R * 4, hipMemcpyDeviceToHost, s_io);
          if (err != hipSuccess) return err;
          bytes_d2h += H * r.R * 4;
          n_d2h += H;
        }
      } else if (!fp.acc_on_device) {
        const float* sn = r.first ? S.n : S.an;
        const float* sml = r.first ? S.ml : S.aml;
        err = copy(PH_D2H, host_n + r.pu * U * nrow_f, sn, r.R * nrow_f * 4, hipMemcpyDeviceToHost, s_io);
        if (err == hipSuccess)
          err = copy(PH_D2H, host_ml + r.pu * U * mlrow_f, sml, r.R * mlrow_f * 4, hipMemcpyDeviceToHost, s_io);
        if (err != hipSuccess) return err;
        bytes_d2h += r.R * (nrow_f + mlrow_f) * 4;
        n_d2h += 2;
      }
      err = step();
      if (err != hipSuccess) return err;
      mw.poll();
    }
    return hipSuccess;
  };
  for (size_t ti = 0; ti < p.tasks.size(); ++ti) {
    const Task& task = p.tasks[ti];
    const int b = static_cast<int>(ti % fp.kv_buffers);
    // keep the host at most two tasks ahead of the GPU
    if (ti >= kTasksAhead) {
      HIP_TRY(hipEventSynchronize(task_done[(ti - kTasksAhead) % (kTasksAhead + 1)]));
      mw.poll();
      if (progress) report(static_cast<int64_t>(ti) - kTasksAhead);
    }
    if (static_cast<int64_t>(ti) >= fp.kv_buffers) HIP_TRY(hipStreamWaitEvent(s_kv, kv_free[b], 0));
    // Chunk reuse: consecutive tasks of one outer task share exactly one inner chunk
    // (a perfect difference set meets its own shift in one residue).  With two staging
    // buffers the previous task's copy of it is still resident, so those rows are copied
    // on the device; every other row comes from the host.  Token lists are in ascending
    // global order, so one sweep over both segment lists finds the shared rows.  The
    // copies stay ordered on the K/V stream: the previous buffer is refilled only after.
    const Task* prev = nullptr;
    if (fp.kv_buffers == 2 && ti > 0 &&
        std::equal(task.ids.begin(), task.ids.end() - 1, p.tasks[ti - 1].ids.begin()))
      prev = &p.tasks[ti - 1];
    size_t ps = 0;
    for (const Segment& g : task.segments) {
      int64_t pos = g.global_start;
      const int64_t end = g.global_start + g.length;
      while (pos < end) {
        while (prev && ps < prev->segments.size() &&
               prev->segments[ps].global_start + prev->segments[ps].length <= pos)
          ++ps;
        const Segment* hit = nullptr;
        int64_t stop = end;
        if (prev && ps < prev->segments.size()) {
          const Segment& s = prev->segments[ps];
          if (s.global_start <= pos)
            hit = &s, stop = std::min(end, s.global_start + s.length);
          else
            stop = std::min(end, s.global_start);
        }
        const int64_t rows = stop - pos, dst = (g.local_offset + pos - g.global_start) * row_in;
        if (hit != nullptr) {
          // on the copy engines: a device copy through compute units would take CUs from the
          // partial kernel running beside it
          const int64_t src = (hit->local_offset + pos - hit->global_start) * row_in;
          HIP_TRY(copy(-1, kst[b] + dst, kst[b ^ 1] + src, rows * row_in, hipMemcpyDeviceToDeviceNoCU, s_kv));
          HIP_TRY(copy(-1, vst[b] + dst, vst[b ^ 1] + src, rows * row_in, hipMemcpyDeviceToDeviceNoCU, s_kv));
          bytes_d2d += 2 * rows * row_in;
        } else {
          HIP_TRY(copy(PH_H2D, kst[b] + dst, k + pos * row_in, rows * row_in, hipMemcpyHostToDevice, s_kv));
          HIP_TRY(copy(PH_H2D, vst[b] + dst, v + pos * row_in, rows * row_in, hipMemcpyHostToDevice, s_kv));
          bytes_h2d += 2 * rows * row_in;
          n_h2d += 2;
        }
        pos = stop;
      }
    }
    HIP_TRY(hipEventRecord(kv_ready[b], s_kv));
    HIP_TRY(hipStreamWaitEvent(s_c, kv_ready[b], 0));
    HIP_TRY(step());

    for (int64_t a = 0; a < tu; ++a, ++blk) {
      const int j = static_cast<int>(blk % 2);
      Slot& S = slot[j];
      const int64_t pu = task.units[a];
      const int64_t R = p.unit_rows(pu);  // U, fewer in the last unit of a padded plan
      if (R == 0) continue;               // a unit of padding only: nothing to compute or copy
      const int visit = task.slot[a];
      const bool first = visit == 0, last = visit == p.visits - 1;
      // the slot's previous block must be copied out first, and so must the previous block
      // when it held this unit's accumulator
      const bool needs_prev = !fp.acc_on_device && !first && last_block[pu] == blk - 1;
      // (the same stream carries this block's inputs, so they follow those copies)
      HIP_TRY(flush_d2h(needs_prev ? blk - 1 : blk - 2));
      // H2D: Q block (+ accumulator block)
      HIP_TRY(copy(PH_H2D, S.q, q + pu * U * row_in, R * row_in, hipMemcpyHostToDevice, s_io));
      bytes_h2d += R * row_in;
      ++n_h2d;
      if (!fp.acc_on_device && !first) {
        HIP_TRY(copy(PH_H2D, S.an, host_n + pu * U * nrow_f, R * nrow_f * 4, hipMemcpyHostToDevice, s_io));
        HIP_TRY(copy(PH_H2D, S.aml, host_ml + pu * U * mlrow_f, R * mlrow_f * 4, hipMemcpyHostToDevice, s_io));
        bytes_h2d += R * (nrow_f + mlrow_f) * 4;
        n_h2d += 2;
      }
      HIP_TRY(hipEventRecord(q_ready[j], s_io));
      HIP_TRY(hipStreamWaitEvent(s_c, q_ready[j], 0));
      HIP_TRY(step());

      // partials of (task, unit)
      float* pn = S.n;
      float* pml = S.ml;
      if (fp.acc_on_device && first) {
        pn = acc_n + pu * U * nrow_f;
        pml = acc_ml + pu * U * mlrow_f;
      }
      AttnLaunch at{};
      at.dtype = p.dtype;
      at.d = p.d;
      at.heads = p.heads;
      at.q = S.q;
      at.k = kst[b];
      at.v = vst[b];
      at.n_out = pn;
      at.ml_out = pml;
      at.items = tabs.stream_items + (int64_t(ti) * tu + a);
      at.runs = tabs.stream_runs;
      at.n_items = 1;
      at.q_len = static_cast<int>(U);
      at.scale_log2 = c2;
      HIP_TRY(tm.begin(PH_ATTN, s_c, tev));
      HIP_TRY(launch_attn(at, s_c));
      HIP_TRY(tm.end(PH_ATTN, s_c));
      ++n_attn;

      // merge into the accumulator (ascending task order per row); the final merge of a
      // unit writes its O block, and its LSE rows into the resident [H][N] array or the
      // slot's [H][unit] block
      MergeLaunch m{};
      m.dtype = p.dtype;
      m.d = p.d;
      m.heads = p.heads;
      m.rows = R;
      m.final_out = last;
      m.o_out = S.o;
      m.lse_out = lse_dev ? lse_dev : S.lse;
      m.lse_stride = lse_dev ? N : U;
      m.lse_row0 = lse_dev ? pu * U : 0;
      bool do_merge = true;
      if (fp.acc_on_device) {
        float* an = acc_n + pu * U * nrow_f;
        float* aml = acc_ml + pu * U * mlrow_f;
        m.n_a = an;
        m.ml_a = aml;
        m.n_b = S.n;
        m.ml_b = S.ml;
        m.nb = first ? 0 : 1;
        m.n_out = an;
        m.ml_out = aml;
        do_merge = !first || last;
      } else {
        if (first) {
          m.n_a = S.n;
          m.ml_a = S.ml;
          m.nb = 0;
          do_merge = last;
        } else {
          m.n_a = S.an;
          m.ml_a = S.aml;
          m.n_b = S.n;
          m.ml_b = S.ml;
          m.nb = 1;
          m.n_out = S.an;
          m.ml_out = S.aml;
        }
      }
      if (do_merge) {
        HIP_TRY(tm.begin(PH_MERGE, s_c, tev));
        HIP_TRY(launch_merge(m, s_c));
        HIP_TRY(tm.end(PH_MERGE, s_c));
        ++n_merge;
      }
      HIP_TRY(hipEventRecord(c_done[j], s_c));
      HIP_TRY(step());

      // D2H of this block: enqueued later, once its kernels have finished (flush_d2h)
      pending.push_back({blk, j, pu, R, first, last});
      if (!fp.acc_on_device && !last) last_block[pu] = blk;
    }
    HIP_TRY(hipEventRecord(kv_free[b], s_c));  // after the task's last launch on s_c
    HIP_TRY(hipEventRecord(task_done[ti % (kTasksAhead + 1)], s_c));
  }
  HIP_TRY(flush_d2h(blk));
  // LSE of every row, in one copy once the last merge has written it
  if (lse != nullptr && lse_dev != nullptr) {
    HIP_TRY(hipEventRecord(all_merged, s_c));
    HIP_TRY(hipEventSynchronize(all_merged));
    HIP_TRY(copy(PH_D2H, lse, lse_dev, H * N * 4, hipMemcpyDeviceToHost, s_io));
    bytes_d2h += H * N * 4;
    ++n_d2h;
  }
  HIP_TRY(hipStreamSynchronize(s_c));
  for (hipStream_t s : res.s) HIP_TRY(hipStreamSynchronize(s));
  mw.poll();
  if (progress)
    for (int64_t t = std::max<int64_t>(0, n_tasks - kTasksAhead); t < n_tasks; ++t) report(t);
  HIP_TRY(hipGetLastError());
  if (canary.on) {
    const std::string bad = canary.check();
    if (!bad.empty()) {
      why = "workspace guard after the " + bad + " was overwritten";
      return CQSA_EHIP;
    }
  }
  if (stats) {
    std::memset(stats, 0, sizeof(*stats));
    stats->t_h2d_ms = tm.total(PH_H2D);
    stats->t_attn_ms = tm.total(PH_ATTN);
    stats->t_merge_ms = tm.total(PH_MERGE);
    stats->t_d2h_ms = tm.total(PH_D2H);
    stats->bytes_h2d = bytes_h2d;
    stats->bytes_d2h = bytes_d2h;
    stats->bytes_d2d = bytes_d2d;
    stats->peak_device_bytes = L.total + tabs.bytes;
    stats->n_attn_launches = n_attn;
    stats->n_merge_launches = n_merge;
    stats->n_h2d_copies = n_h2d;
    stats->n_d2h_copies = n_d2h;
    stats->useful_flop = p.useful_flop();
    stats->levels_used = static_cast<int32_t>(p.ls.size());
    stats->t_total_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
  }
  return CQSA_OK;
}

// The streamed forward with the out-of-memory recovery: when the device workspace of a
// plan cannot be allocated, re-plan one level deeper under the memory the device has
// now (less a 1/16 margin) and run that plan inside the same call; the caller's plan is
// unchanged and the result is the same attention (a different division of it).
cqsa_status forward_stream_recover(const Plan& p, const char* q, const char* k, const char* v, char* o, float* lse,
                                   void* ws, int64_t ws_bytes, hipStream_t caller, cqsa_stats* stats,
                                   std::string& why) {
  {
    const cqsa_status pin = check_pinned({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {lse, "lse"}}, why);
    if (pin != CQSA_OK) return pin;
  }
  const auto t0 = std::chrono::steady_clock::now();
  MemWatch mw;
  mw.begin();
  bool dev_oom = false;
  cqsa_status st = forward_stream(p, q, k, v, o, lse, ws, ws_bytes, caller, stats, mw, dev_oom, why);
  std::unique_ptr<Plan> fb;
  int replans = 0;
  while (st == CQSA_ENOMEM && dev_oom && ws == nullptr) {
    size_t free_b = 0, total_b = 0;
    if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) {
      (void)hipGetLastError();
      return st;
    }
    int64_t budget = static_cast<int64_t>(free_b - free_b / 16);
    const Plan& cur = fb ? *fb : p;
    if (cur.budget > 0) budget = std::min(budget, cur.budget);
    auto next = std::make_unique<Plan>();
    std::string w;
    const cqsa_status fs = fallback_plan(cur, budget, *next, w);
    if (fs != CQSA_OK) {
      why += "; no deeper plan fits the " + std::to_string(budget) + " bytes the device has free: " + w;
      return st;
    }
    if (fb) {
      free_device_tables(*fb);
      free_host_cache(*fb);
    }
    fb = std::move(next);
    ++replans;
    why.clear();
    st = forward_stream(*fb, q, k, v, o, lse, ws, ws_bytes, caller, stats, mw, dev_oom, why);
  }
  if (fb) {
    free_device_tables(*fb);
    free_host_cache(*fb);
  }
  if (st == CQSA_OK && stats) {
    stats->observed_peak_bytes = mw.peak();
    stats->device_free_at_entry = static_cast<int64_t>(mw.free0);
    stats->replans = replans;
    stats->t_total_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
  }
  return st;
}

}  // namespace


// ----------------------------------------------------------------------------------
// backward, host-pinned: Delta of every row first (O and dO streamed through in unit
// blocks), then per task in ascending id: stage Q, K, V, dO of the task's tokens,
// transpose them on the device, gather the task's L and Delta rows, and for each of its
// units run the dQ and dK/dV kernels into a unit block of terms and add the terms into
// the unit's accumulators (device, or pinned host memory with H2D/D2H round trips).  A
// row's first visit stores its terms and later visits add to them -- the order of the
// device path's slot sum -- and its last visit writes the gradient in the input dtype.
// The task staging has one or two sets (the next task is staged while this one runs);
// unit blocks go through a two-slot ring.
// ----------------------------------------------------------------------------------
namespace {

struct BwdStreamRes {
  hipStream_t s[2] = {nullptr, nullptr};  // staging, io
  hipStream_t caller = nullptr;
  std::vector<hipEvent_t> events;
  void* ws = nullptr;
  bool own_ws = false;
  float* host_acc = nullptr;
  float* host_delta = nullptr;  // Delta [H][N] in pinned host memory (host-statistics layouts)
  ~BwdStreamRes() {
    (void)hipStreamSynchronize(caller);
    for (hipStream_t x : s)
      if (x) (void)hipStreamSynchronize(x);
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
    for (hipStream_t x : s)
      if (x) (void)hipStreamDestroy(x);
    if (own_ws && ws) (void)hipFree(ws);
    if (host_acc) (void)hipHostFree(host_acc);
    if (host_delta) (void)hipHostFree(host_delta);
  }
  hipError_t event(hipEvent_t& e) {
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r == hipSuccess) events.push_back(e);
    return r;
  }
};

cqsa_status backward_stream(const Plan& p, const char* q, const char* k, const char* v, const char* o,
                            const float* lse, const char* d_o, char* dq, char* dk, char* dv, void* ws,
                            int64_t ws_bytes, hipStream_t caller, cqsa_stats* stats, std::string& why) {
  {
    const cqsa_status pin = check_pinned({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {lse, "lse"}, {d_o, "d_o"},
                                          {dq, "dq"}, {dk, "dk"}, {dv, "dv"}},
                                         why);
    if (pin != CQSA_OK) return pin;
  }
  const bool causal = (p.flags & CQSA_FLAG_CAUSAL) != 0;
  if (p.bwd_stream_fp.bytes < 0) {
    why = "no streamed backward layout fits the budget of " + std::to_string(p.budget) + " bytes";
    return CQSA_EBUDGET;
  }
  const auto t0 = std::chrono::steady_clock::now();
  MemWatch mw;
  if (stats) mw.begin();
  const bool dev_acc = p.bwd_stream_fp.acc_on_device;
  const int nset = p.bwd_stream_fp.kv_buffers;
  const bool host_stats = p.bwd_host_stats;
  const BwdStreamLayout L = bwd_stream_layout(p, dev_acc, nset, host_stats);
  DeviceTables tabs{};
  cqsa_status st = device_tables(p, tabs, why);
  if (st != CQSA_OK) return st;
  BwdStreamRes R;
  R.caller = caller;
  if (ws == nullptr) {
    HIP_TRY(dev_malloc(&R.ws, L.total));
    R.own_ws = true;
  } else {
    if (ws_bytes < L.total) {
      why = "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(L.total);
      return CQSA_ESMALL;
    }
    R.ws = ws;
  }
  char* cur = static_cast<char*>(R.ws);
  auto take = [&](int64_t bytes) {
    char* r = cur;
    cur += bytes;
    return r;
  };
  const int64_t H = p.heads, D = p.d, U = p.unit, N = p.n, T = p.task_tokens(), e = p.elem_bytes();
  const int64_t row_in = p.row_in_bytes(), hd = H * D;
  // L and Delta of every row: on the device for the call, or (host_stats) L where the caller
  // keeps it and Delta in pinned host memory of the call's own
  float* lse_d = host_stats ? nullptr : reinterpret_cast<float*>(take(L.lse));
  float* delta_d = host_stats ? nullptr : reinterpret_cast<float*>(take(L.delta));
  struct Stage {
    char* t[4];      // Q, K, V, dO of the task
    char* tr[3];     // Q^T, K^T, dO^T
    float* ls;       // the task's L rows [H][T]
    float* ds;       // the task's Delta rows
  } set[2] = {};
  for (int b = 0; b < nset; ++b) {
    Stage& S = set[b];
    for (auto& x : S.t) x = take(L.stage);
    for (auto& x : S.tr) x = L.trans ? take(L.trans) : nullptr;
    S.ls = reinterpret_cast<float*>(take(L.tstat));
    S.ds = reinterpret_cast<float*>(take(L.tstat));
  }
  char** stg = set[0].t;  // phase 0 borrows the first set's Q and dO staging
  struct Slot {
    float* term[3];
    float* temp[3];
    char* out[3];
  } slot[2];
  for (auto& s : slot) {
    for (int g = 0; g < 3; ++g) s.term[g] = reinterpret_cast<float*>(take(L.term));
    for (int g = 0; g < 3; ++g) s.temp[g] = L.temp ? reinterpret_cast<float*>(take(L.temp)) : nullptr;
    for (int g = 0; g < 3; ++g) s.out[g] = take(L.out);
  }
  float* acc[3] = {nullptr, nullptr, nullptr};
  if (dev_acc)
    for (auto& x : acc) x = reinterpret_cast<float*>(take(L.acc));
  float* host_acc[3] = {nullptr, nullptr, nullptr};
  if (!dev_acc) {
    HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&R.host_acc), 3 * N * hd * sizeof(float), hipHostMallocDefault));
    for (int g = 0; g < 3; ++g) host_acc[g] = R.host_acc + g * N * hd;
  }
  char* outs[3] = {dq, dk, dv};
  if (host_stats)
    HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&R.host_delta), H * N * sizeof(float), hipHostMallocDefault));

  for (auto& s : R.s) HIP_TRY(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
  mw.poll();
  // task staging (and the Delta pass) on one stream; a unit's accumulator blocks in and its
  // gradient or accumulator blocks out on another, in the order they are needed; the
  // kernels on the caller's stream
  hipStream_t s_h = R.s[0], s_io = R.s[1], s_c = caller;
  hipEvent_t start, staged, stage_free[2], acc_ready[2], c_done[2];
  HIP_TRY(R.event(start));
  HIP_TRY(R.event(staged));
  for (int i = 0; i < 2; ++i) {
    HIP_TRY(R.event(stage_free[i]));
    HIP_TRY(R.event(acc_ready[i]));
    HIP_TRY(R.event(c_done[i]));
  }
  PhaseTimer tm;
  tm.on = stats != nullptr;
  HIP_TRY(tm.start(caller));
  HIP_TRY(hipEventRecord(start, caller));
  for (hipStream_t s : R.s) HIP_TRY(hipStreamWaitEvent(s, start, 0));
  hipEvent_t tev;
  int64_t bytes_h2d = 0, bytes_d2h = 0, n_attn = 0, n_merge = 0, n_h2d = 0, n_d2h = 0;

  // phase 0: LSE to the device, Delta of every row from O and dO in unit blocks (with
  // host_stats each block of Delta goes back to pinned host memory, through the first
  // staging set's Delta rows, which no task uses yet)
  if (!host_stats) {
    HIP_TRY(tm.begin(PH_H2D, s_h, tev));
    HIP_TRY(hipMemcpyAsync(lse_d, lse, H * N * sizeof(float), hipMemcpyHostToDevice, s_h));
    HIP_TRY(tm.end(PH_H2D, s_h));
    bytes_h2d += H * N * 4;
    ++n_h2d;
  }
  for (int64_t r0 = 0; r0 < N; r0 += U) {
    const int64_t rows = std::min(U, N - r0);
    if (r0 > 0) HIP_TRY(hipStreamWaitEvent(s_h, stage_free[0], 0));
    HIP_TRY(tm.begin(PH_H2D, s_h, tev));
    HIP_TRY(hipMemcpyAsync(stg[0], o + r0 * row_in, rows * row_in, hipMemcpyHostToDevice, s_h));
    HIP_TRY(hipMemcpyAsync(stg[3], d_o + r0 * row_in, rows * row_in, hipMemcpyHostToDevice, s_h));
    HIP_TRY(tm.end(PH_H2D, s_h));
    bytes_h2d += 2 * rows * row_in;
    n_h2d += 2;
    HIP_TRY(hipEventRecord(staged, s_h));
    HIP_TRY(hipStreamWaitEvent(s_c, staged, 0));
    PrepLaunch pr{};
    pr.dtype = p.dtype;
    pr.d = p.d;
    pr.heads = p.heads;
    pr.n = rows;
    pr.o = stg[0];
    pr.d_o = stg[3];
    pr.delta = host_stats ? set[0].ds : delta_d + r0;
    pr.dpitch = host_stats ? U : N;
    HIP_TRY(tm.begin(PH_MERGE, s_c, tev));
    HIP_TRY(launch_bwd_prep(pr, s_c));
    HIP_TRY(tm.end(PH_MERGE, s_c));
    if (host_stats) {
      // rows [r0, r0 + rows) of every head: [H][U] on the device to [H][N] on the host
      HIP_TRY(tm.begin(PH_D2H, s_c, tev));
      HIP_TRY(hipMemcpy2DAsync(R.host_delta + r0, N * 4, set[0].ds, U * 4, rows * 4, H, hipMemcpyDeviceToHost, s_c));
      HIP_TRY(tm.end(PH_D2H, s_c));
      bytes_d2h += H * rows * 4;
      ++n_d2h;
    }
    HIP_TRY(hipEventRecord(stage_free[0], s_c));
  }

  const int64_t tu = p.task_units;
  const float scale = static_cast<float>(1.0 / std::sqrt(double(p.d)));
  std::vector<int64_t> last_block(p.n_units, -4);
  int64_t blk = 0;
  // As in the forward: a block's copies out are enqueued once its kernels have finished
  // (the host stays two blocks ahead), on the stream that then carries the next block's
  // accumulator blocks in.
  struct PendingOut {
    int64_t blk;
    int j;
    int64_t pu, rows;
    bool last;
  };
  std::deque<PendingOut> pending;
  auto flush_out = [&](int64_t upto) -> hipError_t {
    while (!pending.empty() && pending.front().blk <= upto) {
      const PendingOut r = pending.front();
      pending.pop_front();
      hipError_t err = hipEventSynchronize(c_done[r.j]);
      if (err != hipSuccess) return err;
      if (!r.last && dev_acc) continue;
      const Slot& S = slot[r.j];
      err = tm.begin(PH_D2H, s_io, tev);
      for (int g = 0; g < 3 && err == hipSuccess; ++g) {
        if (r.last) {
          err = hipMemcpyAsync(outs[g] + r.pu * U * hd * e, S.out[g], r.rows * hd * e, hipMemcpyDeviceToHost, s_io);
          bytes_d2h += r.rows * hd * e;
        } else {
          err = hipMemcpyAsync(host_acc[g] + r.pu * U * hd, S.temp[g], r.rows * hd * 4, hipMemcpyDeviceToHost, s_io);
          bytes_d2h += r.rows * hd * 4;
        }
        ++n_d2h;
      }
      if (err == hipSuccess) err = tm.end(PH_D2H, s_io);
      if (err != hipSuccess) return err;
    }
    return hipSuccess;
  };
  for (size_t ti = 0; ti < p.tasks.size(); ++ti) {
    const Task& task = p.tasks[ti];
    // stage the task into its set, once the kernels of the set's previous task are done
    const int sb = static_cast<int>(ti % nset);
    Stage& G = set[sb];
    HIP_TRY(hipStreamWaitEvent(s_h, stage_free[sb], 0));
    HIP_TRY(tm.begin(PH_H2D, s_h, tev));
    const char* srcs[4] = {q, k, v, d_o};
    for (const Segment& g : task.segments)
      for (int x = 0; x < 4; ++x) {
        HIP_TRY(hipMemcpyAsync(G.t[x] + g.local_offset * row_in, srcs[x] + g.global_start * row_in, g.length * row_in,
                               hipMemcpyHostToDevice, s_h));
        bytes_h2d += g.length * row_in;
        ++n_h2d;
      }
    if (host_stats) {
      // the task's L and Delta rows, [H][T], from pinned host memory with the staging; the
      // host Delta is complete: this stream waited for the first set's release, recorded
      // after the last Delta block went back, before staging the first task
      for (const Segment& g : task.segments) {
        HIP_TRY(hipMemcpy2DAsync(G.ls + g.local_offset, T * 4, lse + g.global_start, N * 4, g.length * 4, H,
                                 hipMemcpyHostToDevice, s_h));
        HIP_TRY(hipMemcpy2DAsync(G.ds + g.local_offset, T * 4, R.host_delta + g.global_start, N * 4, g.length * 4,
                                 H, hipMemcpyHostToDevice, s_h));
        bytes_h2d += 2 * H * g.length * 4;
        n_h2d += 2;
      }
    }
    HIP_TRY(tm.end(PH_H2D, s_h));
    HIP_TRY(hipEventRecord(staged, s_h));
    HIP_TRY(hipStreamWaitEvent(s_c, staged, 0));
    // the task's L and Delta rows, [H][T]
    HIP_TRY(tm.begin(PH_MERGE, s_c, tev));
    if (!host_stats)
      for (const Segment& g : task.segments) {
        HIP_TRY(hipMemcpy2DAsync(G.ls + g.local_offset, T * 4, lse_d + g.global_start, N * 4, g.length * 4, H,
                                 hipMemcpyDeviceToDevice, s_c));
        HIP_TRY(hipMemcpy2DAsync(G.ds + g.local_offset, T * 4, delta_d + g.global_start, N * 4, g.length * 4, H,
                                 hipMemcpyDeviceToDevice, s_c));
      }
    if (L.trans) {
      PrepLaunch pr{};
      pr.dtype = p.dtype;
      pr.d = p.d;
      pr.heads = p.heads;
      pr.n = T;
      pr.np = L.tnp;
      pr.q = G.t[0];
      pr.k = G.t[1];
      pr.d_o = G.t[3];
      pr.qt = G.tr[0];
      pr.kt = G.tr[1];
      pr.dot = G.tr[2];
      HIP_TRY(launch_bwd_prep(pr, s_c));
    }
    HIP_TRY(tm.end(PH_MERGE, s_c));

    for (int64_t a = 0; a < tu; ++a, ++blk) {
      const int j = static_cast<int>(blk % 2);
      Slot& S = slot[j];
      const int64_t pu = task.units[a];
      const int64_t rows = p.unit_rows(pu);
      if (rows == 0) continue;
      const int visit = task.slot[a];
      const bool first = visit == 0, last = visit == p.visits - 1;
      // the slot's previous block is copied out first, and so is the previous block when it
      // held this unit's accumulator; this block's kernels wait for those copies (they
      // rewrite the slot) and for its own accumulator blocks in
      const bool needs_prev = !dev_acc && !first && last_block[pu] == blk - 1;
      HIP_TRY(flush_out(needs_prev ? blk - 1 : blk - 2));
      if (!dev_acc && !first) {
        // the unit's accumulator blocks back from host memory
        HIP_TRY(tm.begin(PH_H2D, s_io, tev));
        for (int g = 0; g < 3; ++g)
          HIP_TRY(hipMemcpyAsync(S.temp[g], host_acc[g] + pu * U * hd, rows * hd * 4, hipMemcpyHostToDevice, s_io));
        HIP_TRY(tm.end(PH_H2D, s_io));
        bytes_h2d += 3 * rows * hd * 4;
        n_h2d += 3;
      }
      HIP_TRY(hipEventRecord(acc_ready[j], s_io));
      HIP_TRY(hipStreamWaitEvent(s_c, acc_ready[j], 0));
      BwdLaunch b{};
      b.dtype = p.dtype;
      b.d = p.d;
      b.heads = p.heads;
      b.n = T;
      b.np = L.tnp;
      b.q = G.t[0];
      b.k = G.t[1];
      b.v = G.t[2];
      b.d_o = G.t[3];
      b.qt = G.tr[0];
      b.kt = G.tr[1];
      b.dot = G.tr[2];
      b.lse = G.ls;
      b.delta = G.ds;
      b.dq_out = S.term[0];
      b.dk_out = S.term[1];
      b.dv_out = S.term[2];
      b.items = tabs.bstream_items + (int64_t(ti) * tu + a);
      b.runs = tabs.stream_runs;
      b.n_items = 1;
      b.kitems = causal ? tabs.bstream_kitems + (int64_t(ti) * tu + a) : b.items;
      b.kruns = causal ? tabs.bstream_kruns : b.runs;
      b.n_kitems = 1;
      b.causal = causal;
      b.q_len = static_cast<int>(U);
      b.scale = scale;
      HIP_TRY(tm.begin(PH_ATTN, s_c, tev));
      HIP_TRY(launch_bwd_dq(b, s_c));
      HIP_TRY(launch_bwd_dkdv(b, s_c));
      HIP_TRY(tm.end(PH_ATTN, s_c));
      n_attn += 2;
      HIP_TRY(tm.begin(PH_MERGE, s_c, tev));
      for (int g = 0; g < 3; ++g) {
        AccLaunch ac{};
        ac.dtype = p.dtype;
        ac.acc = dev_acc ? acc[g] + pu * U * hd : S.temp[g];
        ac.term = S.term[g];
        ac.count = rows * hd;
        ac.first = first;
        ac.out = last ? S.out[g] : nullptr;
        HIP_TRY(launch_accumulate(ac, s_c));
        ++n_merge;
      }
      HIP_TRY(tm.end(PH_MERGE, s_c));
      HIP_TRY(hipEventRecord(c_done[j], s_c));
      pending.push_back({blk, j, pu, rows, last});
      if (!dev_acc && !last) last_block[pu] = blk;
    }
    HIP_TRY(hipEventRecord(stage_free[sb], s_c));
    mw.poll();
  }
  HIP_TRY(flush_out(blk));
  HIP_TRY(hipStreamSynchronize(s_c));
  for (hipStream_t s : R.s) HIP_TRY(hipStreamSynchronize(s));
  mw.poll();
  HIP_TRY(hipGetLastError());
  if (stats) {
    std::memset(stats, 0, sizeof(*stats));
    stats->t_h2d_ms = tm.total(PH_H2D);
    stats->t_attn_ms = tm.total(PH_ATTN);
    stats->t_merge_ms = tm.total(PH_MERGE);
    stats->t_d2h_ms = tm.total(PH_D2H);
    stats->bytes_h2d = bytes_h2d;
    stats->bytes_d2h = bytes_d2h;
    stats->peak_device_bytes = L.total + tabs.bytes;
    stats->n_attn_launches = n_attn;
    stats->n_merge_launches = n_merge;
    stats->n_h2d_copies = n_h2d;
    stats->n_d2h_copies = n_d2h;
    stats->useful_flop = 2.5 * p.useful_flop();
    stats->observed_peak_bytes = mw.peak();
    stats->device_free_at_entry = static_cast<int64_t>(mw.free0);
    stats->levels_used = static_cast<int32_t>(p.ls.size());
    stats->t_total_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
  }
  return CQSA_OK;
}

}  // namespace

// ----------------------------------------------------------------------------------
// backward, device-resident: prep (Delta, transposed copies), dK/dV terms and dQ terms
// of every (task, unit) into visit slots, then one slot sum per gradient
// ----------------------------------------------------------------------------------
cqsa_status run_backward(const Plan& p, const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* d_o, void* dq, void* dk, void* dv, cqsa_residency res,
                         void* ws, int64_t ws_bytes, hipStream_t stream, cqsa_stats* stats, std::string& why) {
  if (res == CQSA_RES_HOST_PINNED)
    return backward_stream(p, static_cast<const char*>(q), static_cast<const char*>(k), static_cast<const char*>(v),
                           static_cast<const char*>(o), lse, static_cast<const char*>(d_o), static_cast<char*>(dq),
                           static_cast<char*>(dk), static_cast<char*>(dv), ws, ws_bytes, stream, stats, why);
  if (res != CQSA_RES_DEVICE) {
    why = "unknown residency";
    return CQSA_EINVAL;
  }
  if (p.budget > 0 && p.bwd_device_ws + table_bytes(p) > p.budget) {
    why = "device-resident backward needs " + std::to_string(p.bwd_device_ws) + " workspace bytes and " +
          std::to_string(table_bytes(p)) + " descriptor bytes, over the budget";
    return CQSA_EBUDGET;
  }
  MemWatch mw;
  if (stats) mw.begin();
  DeviceTables t{};
  cqsa_status st = device_tables(p, t, why);
  if (st != CQSA_OK) return st;
  const BwdLayout L = bwd_layout(p);
  bool owned = false;
  if (ws == nullptr) {
    HIP_TRY(dev_malloc(&ws, L.total));
    owned = true;
  } else if (ws_bytes < L.total) {
    why = "workspace of " + std::to_string(ws_bytes) + " bytes, need " + std::to_string(L.total);
    return CQSA_ESMALL;
  }
  struct Release {
    void* p;
    hipStream_t s;
    ~Release() {
      if (p) {
        (void)hipStreamSynchronize(s);
        (void)hipFree(p);
      }
    }
  } release{owned ? ws : nullptr, stream};
  char* cur = static_cast<char*>(ws);
  auto take = [&](int64_t bytes) {
    char* r = cur;
    cur += bytes;
    return r;
  };
  float* delta = reinterpret_cast<float*>(take(L.delta));
  void* qt = L.trans ? take(L.trans) : nullptr;
  void* kt = L.trans ? take(L.trans) : nullptr;
  void* dot = L.trans ? take(L.trans) : nullptr;
  float* dq_s = reinterpret_cast<float*>(take(L.slots));
  float* dk_s = reinterpret_cast<float*>(take(L.slots));
  float* dv_s = reinterpret_cast<float*>(take(L.slots));

  PhaseTimer tm;
  tm.on = stats != nullptr;
  hipEvent_t ev;
  const auto t0 = std::chrono::steady_clock::now();
  PrepLaunch pr{};
  pr.dtype = p.dtype;
  pr.d = p.d;
  pr.heads = p.heads;
  pr.n = p.n;
  pr.np = p.bwd_np;
  pr.q = q;
  pr.k = k;
  pr.o = o;
  pr.d_o = d_o;
  pr.delta = delta;
  pr.qt = qt;
  pr.kt = kt;
  pr.dot = dot;
  HIP_TRY(tm.begin(PH_MERGE, stream, ev));
  HIP_TRY(launch_bwd_prep(pr, stream));
  HIP_TRY(tm.end(PH_MERGE, stream));

  BwdLaunch b{};
  b.dtype = p.dtype;
  b.d = p.d;
  b.heads = p.heads;
  b.n = p.n;
  b.np = p.bwd_np;
  b.q = q;
  b.k = k;
  b.v = v;
  b.d_o = d_o;
  b.qt = qt;
  b.kt = kt;
  b.dot = dot;
  b.lse = lse;
  b.delta = delta;
  b.dq_out = dq_s;
  b.dk_out = dk_s;
  b.dv_out = dv_s;
  b.items = t.dev_items;
  b.runs = t.dev_runs;
  b.n_items = static_cast<int>(p.dev_items.size());
  const bool causal = (p.flags & CQSA_FLAG_CAUSAL) != 0;
  b.kitems = causal ? t.dev_kitems : t.dev_items;
  b.kruns = causal ? t.dev_kruns : t.dev_runs;
  b.n_kitems = static_cast<int>(causal ? p.dev_kitems.size() : p.dev_items.size());
  b.causal = causal;
  b.q_len = static_cast<int>(p.unit);
  b.scale = static_cast<float>(1.0 / std::sqrt(double(p.d)));
  HIP_TRY(tm.begin(PH_ATTN, stream, ev));
  HIP_TRY(launch_bwd_dkdv(b, stream));
  HIP_TRY(launch_bwd_dq(b, stream));
  HIP_TRY(tm.end(PH_ATTN, stream));

  SumLaunch sl{};
  sl.dtype = p.dtype;
  sl.d = p.d;
  sl.heads = p.heads;
  sl.rows = p.n;
  sl.stride = p.n * p.heads * int64_t(p.d);
  sl.nslot = static_cast<int>(p.visits);
  HIP_TRY(tm.begin(PH_MERGE, stream, ev));
  const float* ins[3] = {dq_s, dk_s, dv_s};
  void* outs[3] = {dq, dk, dv};
  for (int g = 0; g < 3; ++g) {
    sl.in = ins[g];
    sl.out = outs[g];
    HIP_TRY(launch_sum_slots(sl, stream));
  }
  HIP_TRY(tm.end(PH_MERGE, stream));
  mw.poll();
  if (owned || stats) HIP_TRY(hipStreamSynchronize(stream));
  if (stats) {
    std::memset(stats, 0, sizeof(*stats));
    stats->observed_peak_bytes = mw.peak();
    stats->device_free_at_entry = static_cast<int64_t>(mw.free0);
    stats->levels_used = static_cast<int32_t>(p.ls.size());
    stats->t_total_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    stats->t_attn_ms = tm.total(PH_ATTN);
    stats->t_merge_ms = tm.total(PH_MERGE);
    stats->peak_device_bytes = L.total + t.bytes;
    stats->n_attn_launches = 2;
    stats->n_merge_launches = 4;
    stats->useful_flop = 2.5 * p.useful_flop();
  }
  return CQSA_OK;
}

cqsa_status run_forward(const Plan& p, const void* q, const void* k, const void* v, void* o, float* lse,
                        cqsa_residency res, void* ws, int64_t ws_bytes, hipStream_t stream, cqsa_stats* stats,
                        std::string& why) {
  if (res == CQSA_RES_DEVICE) return forward_device(p, q, k, v, o, lse, ws, ws_bytes, stream, stats, why);
  return forward_stream_recover(p, static_cast<const char*>(q), static_cast<const char*>(k),
                                static_cast<const char*>(v), static_cast<char*>(o), lse, ws, ws_bytes, stream, stats,
                                why);
}

}  // namespace cqsa
