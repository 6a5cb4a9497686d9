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
  const int32_t* order; // device: dispatch order (block b runs entry b: (item * heads + head)
                        // * tiles + tile, or -1), or null for the arithmetic order
  int64_t order_len;    // blocks of the launch when order is given
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

// ---- backward ----
// Delta[h][i] = <dO[i,h,:], O[i,h,:]> (fp32); for bf16 also Q, K, dO transposed to
// [H][d][np] (np >= n rounded up to 64, a multiple of 8; tokens past n are zero).
struct PrepLaunch {
  cqsa_dtype dtype;
  int d, heads;
  int64_t n, np;
  const void* q;
  const void* k;
  const void* o;
  const void* d_o;
  float* delta;        // [H][dpitch] (dpitch 0: n), or null: no Delta
  void* qt;            // bf16 only; null: no transposed copies
  void* kt;
  void* dot;
  int64_t dpitch;
};

// Gradient terms of the pairs the items admit, written to visit slots
// ([slots][n][H][d] fp32, row = item.out_row0 + i).  dK/dV launches treat an item's rows
// as keys and its runs as admitted query runs; dQ launches the other way round.
struct BwdLaunch {
  cqsa_dtype dtype;
  int d, heads;
  int64_t n, np;
  const void* q;       // [n][H][d] bases (rows as in the descriptors)
  const void* k;
  const void* v;
  const void* d_o;
  const void* qt;      // bf16: transposed copies from the prep kernel
  const void* kt;
  const void* dot;
  const float* lse;    // [H][n] natural log
  const float* delta;  // [H][n]
  float* dq_out;
  float* dk_out;
  float* dv_out;
  const WorkItem* items;   // query blocks and their key runs (dQ)
  const KeyRun* runs;
  int n_items;
  const WorkItem* kitems;  // key blocks and their query runs (dK/dV)
  const KeyRun* kruns;
  int n_kitems;
  bool causal;         // runs may carry a causal diagonal (KeyRun::diag >= 0)
  int q_len;           // rows of every item in this launch (upper bound)
  float scale;
};

// out[i] = sum over s < nslot of in[s * stride + i] in slot order, as dtype.
struct SumLaunch {
  cqsa_dtype dtype;
  int d, heads;
  int64_t rows;
  const float* in;
  int64_t stride;      // floats between slots
  int nslot;
  void* out;
};

// acc = term (first) or acc + term; written to acc, or to out (dtype) when out != null.
struct AccLaunch {
  cqsa_dtype dtype;
  float* acc;
  const float* term;
  int64_t count;       // floats (a multiple of 4)
  bool first;
  void* out;
};

int bwd_key_tile(cqsa_dtype dtype);
hipError_t launch_accumulate(const AccLaunch& a, hipStream_t stream);
int bwd_query_tile(cqsa_dtype dtype);
hipError_t launch_bwd_prep(const PrepLaunch& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdLaunch& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdLaunch& a, hipStream_t stream);
hipError_t launch_sum_slots(const SumLaunch& a, hipStream_t stream);

}  // namespace cqsa
