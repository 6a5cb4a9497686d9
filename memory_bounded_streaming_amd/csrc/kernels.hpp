// Launch interface of the HIP kernels (host side).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "../../include/cqsa.h"
#include "descriptors.hpp"

namespace cqsa {

// One launch of the masked attention-partial kernel over n_items query blocks.
struct AttnLaunch {
  cqsa_dtype dtype;
  int d, heads;
  const void* q;        // Q base: query rows are item.q_row0 + i
  const void* k;        // K base: key rows are run.start + j
  const void* v;        // V base, same rows as K
  float* n_out;         // [rows][H][d]   row = item.out_row0 + i
  float* ml_out;        // [rows][H][2]   (m in log2 units, l)
  const WorkItem* items;  // device
  const KeyRun* runs;     // device
  int n_items;
  int q_len;            // rows of every item in this launch
  float scale_log2;     // softmax scale * log2(e)
};

// Merge of (m, l, n) triples: input a, then nb further inputs at b + s*stride,
// folded in that order; writes an accumulator triple or, if final, O and LSE.
struct MergeLaunch {
  cqsa_dtype dtype;
  int d, heads;
  int64_t rows;
  const float* n_a;
  const float* ml_a;
  const float* n_b;
  const float* ml_b;
  int64_t b_stride_n, b_stride_ml;  // elements between further inputs
  int nb;
  bool final_out;
  float* n_out;        // non-final
  float* ml_out;
  void* o_out;         // final: [rows][H][d] in dtype
  float* lse_out;      // final: lse_out[h * lse_stride + lse_row0 + row], may be null
  int64_t lse_stride, lse_row0;
};

// Queries per workgroup of the attention kernel for a dtype (rows of one tile).
int attn_query_tile(cqsa_dtype dtype);

hipError_t launch_attn(const AttnLaunch& a, hipStream_t stream);
hipError_t launch_merge(const MergeLaunch& m, hipStream_t stream);

}  // namespace cqsa
