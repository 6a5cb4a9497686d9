// Device-resident execution and the stream engine behind cqsa_partials / cqsa_merge /
// cqsa_forward.
#pragma once

#include <hip/hip_runtime_api.h>

#include <string>

#include "plan.hpp"

namespace cqsa {

struct DeviceTables {
  const WorkItem* dev_items;
  const KeyRun* dev_runs;
  const WorkItem* stream_items;
  const KeyRun* stream_runs;
  const WorkItem* dev_kitems;  // causal dK/dV tables (empty without causality)
  const KeyRun* dev_kruns;
  const WorkItem* bstream_items;  // streamed backward items (rows in the task staging)
  const WorkItem* bstream_kitems; // causal streamed dK/dV items and runs (task staging rows)
  const KeyRun* bstream_kruns;
  const int32_t* dev_order;       // dispatch order of the device-resident launch, or null
  int64_t dev_order_len;
  int64_t bytes;
};

// Descriptor tables of the plan on the current device (uploaded on first use).
cqsa_status device_tables(const Plan& p, DeviceTables& out, std::string& why);
void free_device_tables(const Plan& p);
// Free the pinned host accumulator a plan keeps between streamed forward calls.
void free_host_cache(const Plan& p);
// Bytes of the plan's descriptor tables on a device.
int64_t table_bytes(const Plan& p);
// Make the next `count` device allocations of the library fail as out of memory.
void set_fail_allocations(int count);

cqsa_status run_partials(const Plan& p, const void* q, const void* k, const void* v, float* n_out,
                         float* ml_out, hipStream_t stream, std::string& why);
// The same launch with the forward descriptor tables (the plan's dev_items and dev_runs,
// and its dispatch order dev_order when it has one) already on the device.
cqsa_status run_partials_with(const Plan& p, const void* q, const void* k, const void* v, float* n_out,
                              float* ml_out, const WorkItem* items, const KeyRun* runs, const int32_t* order,
                              hipStream_t stream, std::string& why);
cqsa_status run_merge(const Plan& p, const float* n_in, const float* ml_in, void* o, float* lse,
                      hipStream_t stream, std::string& why);
// Gradients dQ, dK, dV of the forward for upstream gradient d_o (device-resident).
cqsa_status run_backward(const Plan& p, const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* d_o, void* dq, void* dk, void* dv, cqsa_residency res,
                         void* ws, int64_t ws_bytes, hipStream_t stream, cqsa_stats* stats, std::string& why);
// Device-resident forward with the partial slots and descriptor tables in the library's
// static device array (no allocation); ESMALL when the plan needs more than it holds.
cqsa_status forward_static(const Plan& p, const void* q, const void* k, const void* v, void* o, float* lse,
                           hipStream_t stream, std::string& why);
int64_t static_scratch_capacity();
int64_t static_scratch_need(const Plan& p);
cqsa_status run_forward(const Plan& p, const void* q, const void* k, const void* v, void* o, float* lse,
                        cqsa_residency res, void* ws, int64_t ws_bytes, hipStream_t stream,
                        cqsa_stats* stats, std::string& why);

}  // namespace cqsa
