// Device helpers shared by the forward and backward kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include "descriptors.hpp"

namespace cqsa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef unsigned int u32;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Work of one launch: (item, head) groups of `tiles` workgroups each, item-major, cut
// into equal chunks of at most kChunk tiles (one round of an XCD's 32 CUs).  Workgroups
// are dealt round-robin to the 8 XCDs in launch order (block b runs on XCD b % 8).
// Chunk g goes whole to XCD g % 8, as that XCD's (g / 8)-th chunk: the tiles of a chunk
// share their K/V stream in one L2, and consecutive chunks -- of one large group, or of
// consecutive groups, whose items are ordered heaviest first -- are spread over the
// XCDs, which balances their work.  The grid is 8 * chunk_tiles * ceil(chunks / 8); the
// workgroups past the last chunk, or past the last tile of a shorter final chunk of a
// group, return at once.
constexpr int kChunk = kDispatchChunk;

__host__ __device__ inline int chunks_per_group(int tiles) { return (tiles + kChunk - 1) / kChunk; }
__host__ __device__ inline int chunk_tiles(int tiles) {
  const int per = chunks_per_group(tiles);
  return (tiles + per - 1) / per;
}

inline int64_t group_grid(int64_t groups, int tiles) {
  const int64_t chunks = groups * chunks_per_group(tiles);
  return 8 * int64_t(chunk_tiles(tiles)) * ((chunks + 7) / 8);
}

struct GroupCoord {
  int64_t item;
  int head;
  int tile;
};

__device__ __forceinline__ bool group_coord(int64_t b, int tiles, int heads, int64_t n_items, GroupCoord& c) {
  const int per_group = chunks_per_group(tiles), ct = chunk_tiles(tiles);
  const int64_t i = b >> 3;
  const int64_t g = ((i / ct) << 3) + (b & 7);  // chunk index
  if (g >= n_items * heads * per_group) return false;
  const int tile = static_cast<int>(g % per_group) * ct + static_cast<int>(i % ct);
  if (tile >= tiles) return false;
  const int64_t gh = g / per_group;
  c.tile = tile;
  c.head = static_cast<int>(gh % heads);
  c.item = gh / heads;
  return true;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Cursor over the tiles of an item's key runs.  The current run's start and length
// are kept in (scalar) registers and reloaded only when the cursor enters a new run.
// On a causal diagonal run (diag >= 0) the run is cut after the last key any query
// of the workgroup can see: key j is visible to query i only if j <= diag + i, and the
// workgroup's queries end before qhi.
struct TileCursor {
  int run;        // index of the current run (nrun when exhausted)
  int k0;         // first key of the tile within the run
  int len;        // length of the current run (cut as above on a diagonal run)
  int diag;       // the run's diagonal offset, -1 if every key is visible
  int64_t start;  // first key row of the current run
};

__device__ __forceinline__ void cursor_settle(TileCursor& c, const KeyRun* runs, int nrun, int qhi) {
  while (c.run < nrun) {
    // The run table is read-only and the index wave-uniform: reading it through the
    // constant address space at a lane-0 address makes these scalar loads, which keep
    // the vector-memory counter free for the tile loads.
    const uint64_t ra = reinterpret_cast<uint64_t>(runs + c.run);
    const uint64_t ru = (uint64_t(__builtin_amdgcn_readfirstlane(unsigned(ra >> 32))) << 32) |
                        unsigned(__builtin_amdgcn_readfirstlane(unsigned(ra)));
    const __attribute__((address_space(4))) KeyRun* rp = (const __attribute__((address_space(4))) KeyRun*)(ru);
    const int64_t rstart = rp->start;
    const int rlen = rp->len, rdiag = rp->diag;
    const int len = rdiag >= 0 ? min(rlen, rdiag + qhi) : rlen;
    if (len > 0) {
      c.start = rstart;
      c.len = len;
      c.diag = rdiag;
      return;
    }
    ++c.run;
  }
  c.len = 0;
  c.diag = -1;
  c.start = 0;
}

__device__ __forceinline__ TileCursor cursor_begin(const KeyRun* runs, int nrun, int qhi) {
  TileCursor c{0, 0, 0, -1, 0};
  cursor_settle(c, runs, nrun, qhi);
  return c;
}

__device__ __forceinline__ void cursor_next(TileCursor& c, const KeyRun* runs, int nrun, int kt, int qhi) {
  c.k0 += kt;
  if (c.k0 >= c.len) {
    ++c.run;
    c.k0 = 0;
    cursor_settle(c, runs, nrun, qhi);
  }
}

// Stores of four fp32 values as fp32, or as bf16 rounded to nearest even.
__device__ __forceinline__ void store_out(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

__device__ __forceinline__ u32 bf16_rne(float x) {
  const u32 u = __builtin_bit_cast(u32, x);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);  // inf / nan
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void store_out(u16* p, float4 v) {
  const u32 a = bf16_rne(v.x) | (bf16_rne(v.y) << 16);
  const u32 b = bf16_rne(v.z) | (bf16_rne(v.w) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
}

}  // namespace dev
}  // namespace cqsa
