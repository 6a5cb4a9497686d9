// Descriptor records shared by the host planner and the HIP kernels.
// Plain structs with fixed layout; no HIP or host-only types.
#pragma once

#include <cstdint>

namespace cqsa {

// A contiguous run of admitted keys, in token rows of the K/V base the kernel reads.
struct KeyRun {
  int64_t start;  // first key row
  int32_t len;    // number of keys (may be any positive count)
  int32_t diag;   // -1: every row of the run pairs with every row of the item.  >= 0:
                  // the causal diagonal run.  In the tables whose items are query
                  // blocks (forward, dQ), key j of the run is visible to query i of the
                  // item only if j <= diag + i; in the key-block table of a causal dK/dV
                  // pass, query j of the run sees key i of the item only if j >= diag + i
};

// One query block and its admitted keys.
struct WorkItem {
  int64_t q_row0;    // first query row in the Q base
  int64_t out_row0;  // first row of the block in the (n, ml) output arrays
  int32_t q_len;     // query rows in the block
  int32_t run0;      // first KeyRun of this item
  int32_t nrun;      // number of KeyRuns
  int32_t keys;      // total admitted keys (for ordering only)
};

// Launch shape of the attention-partial kernel, shared by the kernel and the planner's
// dispatch order: query rows and keys per workgroup tile (bf16 / float32), and the most
// workgroups of one (item, head) group that go to one XCD together (one round of its 32 CUs).
constexpr int kAttnQueryTileBf16 = 256, kAttnQueryTileF32 = 64;
constexpr int kAttnKeyTileBf16 = 64, kAttnKeyTileF32 = 32;
constexpr int kDispatchChunk = 32;
// Largest dispatch table the planner builds (entries of 4 bytes); a launch with more
// workgroups keeps the arithmetic order.
constexpr int64_t kMaxDispatchEntries = int64_t(1) << 20;

static_assert(sizeof(KeyRun) == 16, "KeyRun layout");
static_assert(sizeof(WorkItem) == 32, "WorkItem layout");

}  // namespace cqsa
