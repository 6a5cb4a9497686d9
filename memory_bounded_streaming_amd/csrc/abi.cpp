// extern "C" entry points of libcqsa.so (declared and documented in include/cqsa.h).
// Every call validates its arguments, converts failures into a cqsa_status and keeps a
// thread-local message; no exception crosses the boundary.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <exception>
#include <new>
#include <string>

#include "../../include/cqsa.h"
#include "engine.hpp"
#include "plan.hpp"

struct cqsa_plan {
  cqsa::Plan p;
};

namespace {

thread_local std::string g_last_error;

cqsa_status fail(cqsa_status s, const std::string& why) {
  g_last_error = why;
  return s;
}

cqsa_status ok() {
  g_last_error.clear();
  return CQSA_OK;
}

// The kernels move tensor rows in 16-byte vectors; the row stride H*d is a multiple of
// 128 bytes, so the base addresses decide the alignment.
bool aligned(const void* p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned(p, 16)) return false;
  return true;
}

constexpr const char* kAlignWhy = "device tensors and workspaces must start on a 16-byte boundary (lse on a 4-byte one)";

// CQSA_FLAG_FREE_BUDGET: the budget is the current device's free memory less the margin
// the caller passed as budget_bytes.
cqsa_status free_budget(uint32_t flags, int64_t& budget) {
  if (!(flags & CQSA_FLAG_FREE_BUDGET)) return CQSA_OK;
  if (budget < 0) return fail(CQSA_EINVAL, "the margin (budget_bytes) must be >= 0");
  size_t free_b = 0, total_b = 0;
  const hipError_t e = hipMemGetInfo(&free_b, &total_b);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(CQSA_EHIP, std::string("hipMemGetInfo: ") + hipGetErrorString(e));
  }
  if (static_cast<int64_t>(free_b) <= budget)
    return fail(CQSA_EBUDGET, "the margin of " + std::to_string(budget) + " bytes exceeds the " +
                                  std::to_string(free_b) + " bytes free on the device");
  budget = static_cast<int64_t>(free_b) - budget;
  return CQSA_OK;
}

template <typename F>
cqsa_status guarded(F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return fail(CQSA_ENOMEM, "host allocation failed");
  } catch (const std::exception& e) {
    return fail(CQSA_EINVAL, std::string("internal error: ") + e.what());
  } catch (...) {
    return fail(CQSA_EINVAL, "internal error");
  }
}

}  // namespace

extern "C" {

const char* cqsa_version(void) { return "cqsa 0.1.0 (gfx950)"; }

const char* cqsa_status_string(cqsa_status s) {
  switch (s) {
    case CQSA_OK: return "CQSA_OK";
    case CQSA_EINVAL: return "CQSA_EINVAL: invalid argument";
    case CQSA_ENOSET: return "CQSA_ENOSET: no perfect difference set for this l";
    case CQSA_EDIVIDE: return "CQSA_EDIVIDE: N does not divide into the unit grid";
    case CQSA_EBUDGET: return "CQSA_EBUDGET: no staging mode fits the memory budget";
    case CQSA_EHIP: return "CQSA_EHIP: HIP runtime error";
    case CQSA_ENOMEM: return "CQSA_ENOMEM: allocation failed";
    case CQSA_ESMALL: return "CQSA_ESMALL: buffer too small";
  }
  return "unknown cqsa_status";
}

const char* cqsa_last_error(void) { return g_last_error.c_str(); }

cqsa_status cqsa_difference_set(int32_t l, int32_t* out, int32_t cap) {
  return guarded([&]() -> cqsa_status {
    if (out == nullptr || cap < l) return fail(CQSA_EINVAL, "out must hold at least l values");
    std::vector<int> d;
    std::string why;
    const cqsa_status s = cqsa::difference_set(l, d, why);
    if (s != CQSA_OK) return fail(s, why);
    for (size_t i = 0; i < d.size(); ++i) out[i] = d[i];
    return ok();
  });
}

cqsa_status cqsa_plan_create(int64_t n, int32_t heads, int32_t head_dim, cqsa_dtype dtype, const int32_t* l_levels,
                             int32_t n_levels, int64_t budget_bytes, uint32_t flags, cqsa_plan** out) {
  return guarded([&]() -> cqsa_status {
    if (out == nullptr) return fail(CQSA_EINVAL, "out is NULL");
    *out = nullptr;
    const cqsa_status fb = free_budget(flags, budget_bytes);
    if (fb != CQSA_OK) return fb;
    auto* plan = new cqsa_plan();
    std::string why;
    const cqsa_status s = cqsa::build_plan(n, heads, head_dim, dtype, l_levels, n_levels, budget_bytes, flags,
                                           plan->p, why);
    if (s != CQSA_OK) {
      delete plan;
      return fail(s, why);
    }
    *out = plan;
    return ok();
  });
}

cqsa_status cqsa_plan_info_get(const cqsa_plan* plan, cqsa_plan_info* out) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || out == nullptr) return fail(CQSA_EINVAL, "NULL argument");
    const cqsa::Plan& p = plan->p;
    std::memset(out, 0, sizeof(*out));
    out->n_tokens = p.n;
    out->heads = p.heads;
    out->head_dim = p.d;
    out->dtype = p.dtype;
    out->levels = static_cast<int32_t>(p.ls.size());
    for (size_t k = 0; k < p.ls.size(); ++k) {
      out->c[k] = p.cs[k];
      out->l[k] = p.ls[k];
    }
    out->n_tasks = static_cast<int64_t>(p.tasks.size());
    out->unit_tokens = p.unit;
    out->n_units = p.n_units;
    out->visits = p.visits;
    out->task_tokens = p.task_tokens();
    out->budget_bytes = p.budget;
    out->stream_mode = p.stream_fp.acc_on_device ? (p.stream_fp.kv_buffers == 2 ? CQSA_MODE_DEVICE_ACC_KV2 : CQSA_MODE_DEVICE_ACC_KV1)
                                                 : (p.stream_fp.kv_buffers == 2 ? CQSA_MODE_HOST_ACC_KV2 : CQSA_MODE_HOST_ACC_KV1);
    out->kv_buffers = p.stream_fp.kv_buffers;
    out->stream_workspace_bytes = p.stream_fp.bytes;
    out->device_workspace_bytes = p.device_ws;
    out->host_acc_bytes = p.host_acc_bytes;
    out->useful_flop = p.useful_flop();
    out->padded_tokens = p.n_pad;
    const cqsa::Footprint& b = p.bwd_stream_fp;
    out->bwd_stream_mode = b.bytes < 0 ? 0
                           : b.acc_on_device ? (b.kv_buffers == 2 ? CQSA_MODE_DEVICE_ACC_KV2 : CQSA_MODE_DEVICE_ACC_KV1)
                                             : (b.kv_buffers == 2 ? CQSA_MODE_HOST_ACC_KV2 : CQSA_MODE_HOST_ACC_KV1);
    out->bwd_host_stats = p.bwd_host_stats ? 1 : 0;
    out->bwd_stream_workspace_bytes = b.bytes;
    return ok();
  });
}

cqsa_status cqsa_plan_schedule(const cqsa_plan* plan, int64_t* buf, int64_t cap, int64_t* needed) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || needed == nullptr) return fail(CQSA_EINVAL, "NULL argument");
    const auto& s = plan->p.schedule;
    *needed = static_cast<int64_t>(s.size());
    if (cap == 0) return ok();
    if (buf == nullptr || cap < *needed) return fail(CQSA_ESMALL, "schedule buffer too small");
    std::memcpy(buf, s.data(), s.size() * sizeof(int64_t));
    return ok();
  });
}

cqsa_status cqsa_plan_coverage(const cqsa_plan* plan, int32_t* table, int64_t cap, int64_t* needed) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || needed == nullptr) return fail(CQSA_EINVAL, "NULL argument");
    const cqsa::Plan& p = plan->p;
    const int64_t u = p.n_units;
    *needed = u * u;
    if (cap == 0) return ok();
    if (table == nullptr || cap < *needed) return fail(CQSA_ESMALL, "coverage buffer too small");
    for (int64_t i = 0; i < u * u; ++i) table[i] = -1;
    for (const cqsa::Task& t : p.tasks)
      for (size_t a = 0; a < t.units.size(); ++a)
        for (const cqsa::UnitRun& r : t.runs[a])
          for (int32_t b = r.start; b < r.start + r.count; ++b) {
            int32_t& cell = table[t.units[a] * u + t.units[b]];
            cell = cell == -1 ? static_cast<int32_t>(t.tid) : -2;  // -2 would mark a doubly owned pair
          }
    return ok();
  });
}

void cqsa_plan_destroy(cqsa_plan* plan) {
  if (plan == nullptr) return;
  try {
    cqsa::free_device_tables(plan->p);
    cqsa::free_host_cache(plan->p);
  } catch (...) {
  }
  delete plan;
}

cqsa_status cqsa_workspace_size(const cqsa_plan* plan, cqsa_residency res, int64_t* bytes) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || bytes == nullptr) return fail(CQSA_EINVAL, "NULL argument");
    if (res == CQSA_RES_DEVICE)
      *bytes = plan->p.device_ws;
    else if (res == CQSA_RES_HOST_PINNED)
      *bytes = plan->p.stream_fp.bytes;
    else
      return fail(CQSA_EINVAL, "unknown residency");
    return ok();
  });
}

cqsa_status cqsa_partials(const cqsa_plan* plan, const void* q, const void* k, const void* v, float* n_out,
                          float* ml_out, void* stream) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || q == nullptr || k == nullptr || v == nullptr || n_out == nullptr || ml_out == nullptr)
      return fail(CQSA_EINVAL, "NULL argument");
    if (!aligned16({q, k, v, n_out, ml_out})) return fail(CQSA_EINVAL, kAlignWhy);
    std::string why;
    const cqsa_status s = cqsa::run_partials(plan->p, q, k, v, n_out, ml_out, static_cast<hipStream_t>(stream), why);
    return s == CQSA_OK ? ok() : fail(s, why);
  });
}

cqsa_status cqsa_merge(const cqsa_plan* plan, const float* n_in, const float* ml_in, void* o, float* lse,
                       void* stream) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || n_in == nullptr || ml_in == nullptr || o == nullptr)
      return fail(CQSA_EINVAL, "NULL argument");
    if (!aligned16({n_in, ml_in, o}) || !aligned(lse, 4)) return fail(CQSA_EINVAL, kAlignWhy);
    std::string why;
    const cqsa_status s = cqsa::run_merge(plan->p, n_in, ml_in, o, lse, static_cast<hipStream_t>(stream), why);
    return s == CQSA_OK ? ok() : fail(s, why);
  });
}

cqsa_status cqsa_forward(const cqsa_plan* plan, const void* q, const void* k, const void* v, void* o, float* lse,
                         cqsa_residency res, void* workspace, int64_t workspace_bytes, void* stream,
                         cqsa_stats* stats) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || q == nullptr || k == nullptr || v == nullptr || o == nullptr)
      return fail(CQSA_EINVAL, "NULL argument");
    if (res != CQSA_RES_DEVICE && res != CQSA_RES_HOST_PINNED) return fail(CQSA_EINVAL, "unknown residency");
    if (workspace != nullptr && workspace_bytes <= 0) return fail(CQSA_EINVAL, "workspace size must be positive");
    if (!aligned(workspace, 16) ||
        (res == CQSA_RES_DEVICE && (!aligned16({q, k, v, o}) || !aligned(lse, 4))))
      return fail(CQSA_EINVAL, kAlignWhy);
    std::string why;
    const cqsa_status s = cqsa::run_forward(plan->p, q, k, v, o, lse, res, workspace, workspace_bytes,
                                            static_cast<hipStream_t>(stream), stats, why);
    return s == CQSA_OK ? ok() : fail(s, why);
  });
}

cqsa_status cqsa_forward_noalloc(const cqsa_plan* plan, const void* q, const void* k, const void* v, void* o,
                                 float* lse, void* stream) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || q == nullptr || k == nullptr || v == nullptr || o == nullptr)
      return fail(CQSA_EINVAL, "NULL argument");
    if (!aligned16({q, k, v, o}) || !aligned(lse, 4)) return fail(CQSA_EINVAL, kAlignWhy);
    std::string why;
    const cqsa_status s = cqsa::forward_static(plan->p, q, k, v, o, lse, static_cast<hipStream_t>(stream), why);
    return s == CQSA_OK ? ok() : fail(s, why);
  });
}

cqsa_status cqsa_backward_workspace_size(const cqsa_plan* plan, cqsa_residency res, int64_t* bytes) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || bytes == nullptr) return fail(CQSA_EINVAL, "NULL argument");
    if (res == CQSA_RES_HOST_PINNED) {
      if (plan->p.bwd_stream_fp.bytes < 0) return fail(CQSA_EBUDGET, "no streamed backward layout fits the budget");
      *bytes = plan->p.bwd_stream_fp.bytes;
      return ok();
    }
    if (res != CQSA_RES_DEVICE) return fail(CQSA_EINVAL, "unknown residency");
    *bytes = plan->p.bwd_device_ws;
    return ok();
  });
}

cqsa_status cqsa_backward(const cqsa_plan* plan, const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* d_o, void* dq, void* dk, void* dv, cqsa_residency res,
                          void* workspace, int64_t workspace_bytes, void* stream, cqsa_stats* stats) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
        d_o == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
      return fail(CQSA_EINVAL, "NULL argument");
    if (res != CQSA_RES_DEVICE && res != CQSA_RES_HOST_PINNED) return fail(CQSA_EINVAL, "unknown residency");
    if (workspace != nullptr && workspace_bytes <= 0) return fail(CQSA_EINVAL, "workspace size must be positive");
    if (!aligned(workspace, 16) ||
        (res == CQSA_RES_DEVICE && (!aligned16({q, k, v, o, d_o, dq, dk, dv}) || !aligned(lse, 4))))
      return fail(CQSA_EINVAL, kAlignWhy);
    std::string why;
    const cqsa_status s = cqsa::run_backward(plan->p, q, k, v, o, lse, d_o, dq, dk, dv, res, workspace,
                                             workspace_bytes, static_cast<hipStream_t>(stream), stats, why);
    return s == CQSA_OK ? ok() : fail(s, why);
  });
}

cqsa_status cqsa_plan_estimate(int64_t n, int32_t heads, int32_t head_dim, cqsa_dtype dtype,
                               const int32_t* l_levels, int32_t n_levels, int64_t budget_bytes, uint32_t flags,
                               const cqsa_rates* rates, cqsa_estimate* out) {
  return guarded([&]() -> cqsa_status {
    if (rates == nullptr || out == nullptr) return fail(CQSA_EINVAL, "NULL argument");
    const cqsa_status fb = free_budget(flags, budget_bytes);
    if (fb != CQSA_OK) return fb;
    std::string why;
    const cqsa_status s = cqsa::estimate_plan(n, heads, head_dim, dtype, l_levels, n_levels, budget_bytes, flags,
                                              *rates, *out, why);
    return s == CQSA_OK ? ok() : fail(s, why);
  });
}

cqsa_status cqsa_plan_fallback(const cqsa_plan* plan, int64_t budget_bytes, cqsa_plan** out) {
  return guarded([&]() -> cqsa_status {
    if (plan == nullptr || out == nullptr) return fail(CQSA_EINVAL, "NULL argument");
    *out = nullptr;
    auto* next = new cqsa_plan();
    std::string why;
    const cqsa_status s = cqsa::fallback_plan(plan->p, budget_bytes, next->p, why);
    if (s != CQSA_OK) {
      delete next;
      return fail(s, why);
    }
    *out = next;
    return ok();
  });
}

cqsa_status cqsa_debug_fail_allocations(int32_t count) {
  if (count < 0) return fail(CQSA_EINVAL, "count must be >= 0");
  cqsa::set_fail_allocations(count);
  return ok();
}

}  // extern "C"
