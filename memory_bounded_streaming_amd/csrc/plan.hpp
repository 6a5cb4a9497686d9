// Host CQS planner: difference sets, task construction over levels, the CQS Mask,
// coverage table, canonical schedule record, kernel descriptor tables and the
// device-memory footprint model.  Pure C++17, no HIP dependency.
#pragma once

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/cqsa.h"
#include "descriptors.hpp"

namespace cqsa {

struct Error {
  cqsa_status status;
  std::string msg;
};

// Lexicographically smallest perfect difference set with {0,1} (l >= 2) or {0} (l = 1).
cqsa_status difference_set(int l, std::vector<int>& out, std::string& why);

struct Segment {     // a globally contiguous piece of a task's token list
  int64_t global_start, length, local_offset;  // tokens
};

struct UnitRun {     // admitted keys of one query unit, task-local units
  int32_t start, count;
};

struct Task {
  int64_t tid = 0;
  std::vector<int> ids;                 // per-level subsequence index
  std::vector<int64_t> units;           // global unit of each local unit
  std::vector<Segment> segments;
  std::vector<std::vector<UnitRun>> runs;  // per local query unit
  std::vector<int32_t> slot;            // visit ordinal of this task for each local unit
  int64_t admitted_units = 0;           // admitted (query unit, key unit) pairs
};

struct Footprint {
  bool acc_on_device;
  int kv_buffers;
  int64_t bytes;
};

struct Plan {
  int64_t n = 0;                        // real tokens
  int64_t n_pad = 0;                    // tokens the division covers (unit * n_units >= n)
  int heads = 0, d = 0;
  cqsa_dtype dtype = CQSA_BF16;
  std::vector<int> ls, cs;
  std::vector<std::vector<int>> sets;
  int64_t unit = 0, n_units = 0, visits = 0, task_units = 0;
  int64_t budget = 0;
  uint32_t flags = 0;
  std::vector<Task> tasks;

  std::vector<int64_t> schedule;        // canonical record
  std::vector<int32_t> coverage;        // [U*U]

  // kernel descriptors
  std::vector<WorkItem> dev_items;      // all (task, unit) items, global coordinates
  std::vector<KeyRun> dev_runs;
  // causal plans: dispatch order of the device-resident partial launch (entry b = the
  // workgroup block b runs, (item * heads + head) * tiles + tile, or -1); empty otherwise
  std::vector<int32_t> dev_order;
  std::vector<WorkItem> stream_items;   // item (t, a) at index t*task_units + a, block coordinates
  std::vector<KeyRun> stream_runs;
  // causal dK/dV: (task, key unit) items whose runs are the admitted query units at or
  // after the key unit (without causality the mask is symmetric: dev_items serve)
  std::vector<WorkItem> dev_kitems;
  std::vector<KeyRun> dev_kruns;
  // streamed backward: item (t, a) at index t*task_units + a, rows in the task's staging
  // (q_row0 = a * unit), outputs in a unit block (out_row0 = 0); runs are stream_runs
  std::vector<WorkItem> bstream_items;
  // causal streamed dK/dV: the key-block tables in the same task-local coordinates
  std::vector<WorkItem> bstream_kitems;
  std::vector<KeyRun> bstream_kruns;

  Footprint stream_fp{};
  int64_t device_ws = 0;                // slots bytes of the device-resident path
  int64_t bwd_np = 0;                   // row pitch (tokens) of the backward's transposed copies
  int64_t bwd_device_ws = 0;            // workspace bytes of the device-resident backward
  Footprint bwd_stream_fp{};            // streamed backward mode (bytes < 0: none fits the budget)
  bool bwd_host_stats = false;          // streamed backward keeps L and Delta in pinned host memory
  int64_t host_acc_bytes = 0;

  // device copies of the descriptor tables, uploaded lazily per device
  mutable std::mutex dev_mu;
  mutable std::vector<std::pair<int, void*>> dev_tables;  // (device, allocation)
  // pinned host accumulator of the streamed forward, kept between calls; a call that finds
  // it in use (another thread's call on the same plan) allocates its own
  mutable std::mutex host_mu;
  mutable void* host_acc_cache = nullptr;
  mutable int64_t host_acc_cache_bytes = 0;
  mutable bool host_acc_busy = false;

  int64_t elem_bytes() const { return dtype == CQSA_BF16 ? 2 : 4; }
  int64_t row_in_bytes() const { return int64_t(heads) * d * elem_bytes(); }
  int64_t row_part_bytes() const { return int64_t(heads) * (d + 2) * 4; }
  int64_t row_out_bytes() const { return int64_t(heads) * (d * elem_bytes() + 4); }
  int64_t task_tokens() const { return task_units * unit; }
  // useful attention FLOP: 4 d H per (query, key) pair attended
  double useful_flop() const {
    const double nn = (flags & CQSA_FLAG_CAUSAL) ? 0.5 * double(n) * double(n + 1) : double(n) * double(n);
    return 4.0 * nn * d * heads;
  }
  // real query rows of global unit u (0 for a unit that is all padding)
  int64_t unit_rows(int64_t u) const { return std::max<int64_t>(0, std::min(unit, n - u * unit)); }
};

// Byte size of each piece of the device-resident backward's workspace, in carve order.
struct BwdLayout {
  int64_t delta;        // [H][N] fp32
  int64_t trans;        // one transposed copy [H][d][np] bf16 (0 for fp32 inputs)
  int64_t slots;        // one gradient's visit slots [V][N][H][d] fp32
  int64_t total;        // delta + 3 trans + 3 slots
};
BwdLayout bwd_layout(const Plan& p);

// Byte size of each piece of the streamed backward's workspace, in carve order.
struct BwdStreamLayout {
  int64_t lse, delta;     // [H][N] fp32 each, resident for the call (0 with host_stats)
  int64_t stage;          // one staged tensor of a task (Q, K, V or dO): task_tokens rows
  int64_t trans;          // one transposed staged tensor [H][d][tnp] bf16 (0 for fp32)
  int64_t tstat;          // the task's L or Delta rows [H][task_tokens] fp32
  int64_t term;           // one gradient's terms of a unit [U][H][d] fp32 (per ring slot)
  int64_t temp;           // host accumulator block [U][H][d] fp32 (per ring slot; 0 on device)
  int64_t out;            // one output block [U][H][d] dtype (per ring slot)
  int64_t acc;            // one device accumulator [N][H][d] fp32 (0 with the host one)
  int64_t tnp;            // row pitch of the transposed staging (tokens)
  int sets;               // task staging sets (2: the next task is staged during this one)
  bool host_stats;        // L and Delta of every row stay in pinned host memory; each task's
                          // rows are gathered from there with its staging
  int64_t total;
};
BwdStreamLayout bwd_stream_layout(const Plan& p, bool acc_on_device, int stage_sets, bool host_stats = false);

// Byte size of each piece of the streamed path's workspace, in the order it is carved.
struct StreamLayout {
  int64_t kv_stage;     // one K or V staging buffer (task_tokens rows)
  int64_t q_blk, n_blk, ml_blk, o_blk;  // per ring slot (unit rows)
  int64_t lse_blk;      // per ring slot: LSE [H][unit] of a finished block (0 when resident)
  int64_t lse_all;      // LSE [H][N] fp32 resident for the call and copied back once, when
                        // it is at most 1/16 of the budget (0 otherwise)
  int64_t acc_n, acc_ml; // device accumulator (0 when on host)
  int64_t total;
};
StreamLayout stream_layout(const Plan& p, bool acc_on_device, int kv_buffers);

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Device bytes of a built plan's descriptor tables (0 for a plan whose tasks were not
// built); every budget test adds them to the layout's workspace.
int64_t descriptor_bytes(const Plan& p);

// Build a plan; on failure returns the status and fills why.
cqsa_status build_plan(int64_t n, int heads, int d, cqsa_dtype dtype, const int32_t* ls,
                       int n_levels, int64_t budget, uint32_t flags, Plan& out, std::string& why);

// The out-of-memory fallback of `p`: one level deeper (repeating the innermost l, 3 for
// an undivided plan), padded when N no longer divides, under `budget`; further levels
// while no staging mode fits (cqsa_plan_fallback).
cqsa_status fallback_plan(const Plan& p, int64_t budget, Plan& out, std::string& why);

// Closed-form dry run of the streamed forward (cqsa_plan_estimate).
cqsa_status estimate_plan(int64_t n, int heads, int d, cqsa_dtype dtype, const int32_t* ls, int n_levels,
                          int64_t budget, uint32_t flags, const cqsa_rates& r, cqsa_estimate& out,
                          std::string& why);

}  // namespace cqsa
