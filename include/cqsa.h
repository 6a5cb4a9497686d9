/*
 * cqsa.h -- C ABI of the Stream-CQSA forward library (libcqsa.so, MI355X / gfx950).
 *
 * The method (sources are the pages describing it):
 *   - "Stream-CQSA: Exact Out-of-Memory Recovery for Attention" (arXiv 2604.20819),
 *     abstract: an infeasible attention call is partitioned recursively into
 *     independent subsequence tasks; each runs an inner attention kernel and the
 *     local statistics are recomposed into the exact full output.
 *   - "Stream-CQSA: Breaking the Billion-Token Barrier on a Single GPU" (wispaper
 *     explainer), section "The 'CQS Divide': Attention as a Steiner System":
 *     N tokens -> c = l(l-1)+1 chunks -> c subsequences of l chunks, every chunk
 *     pair exactly once; section "The Recursive Benefit": divide again until a
 *     task fits the memory budget; section "Implementation: From High-Level Logic
 *     to GPU Kernels": the CQS Mask, each task's Q, K and V moved to the device,
 *     per-task softmax sums, aggregation in host memory.
 *   - Lattice summary of arXiv:2604.20819: subproblems that fit arbitrary memory
 *     budgets; recomposition equals full-sequence attention.
 *
 * Conventions for every call
 *   - Tensors are token-major [N, H, d] (batch 1), row stride H*d elements.
 *     dtype CQSA_BF16 = bfloat16 (2 bytes), CQSA_F32 = float32.
 *   - Attention is over all N keys (non-causal) unless the plan was created with
 *     CQSA_FLAG_CAUSAL (row i then attends keys j <= i); softmax scale 1/sqrt(d).
 *   - Every call returns a cqsa_status; 0 is success.  On failure nothing is
 *     guaranteed about outputs, and cqsa_last_error() returns a thread-local
 *     message.  No C++ exception crosses this boundary.
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *   - Device pointers must be on the current HIP device.  Device tensors (and any
 *     workspace) must start on a 16-byte boundary, an LSE array on a 4-byte one
 *     (rows are moved in 16-byte vectors; every row stride is a multiple of 128 bytes);
 *     a misaligned pointer is EINVAL.  Host-pinned tensors have no such requirement.
 */
#ifndef CQSA_H
#define CQSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums of this header are int-sized in C.  Compiled as C++ they take int as their
 * fixed underlying type, so every int a caller passes is a value of the enum type (a
 * value outside the listed ones is then rejected with CQSA_EINVAL rather than being a
 * value the type cannot hold); the layout and the calling convention are the same. */
#ifdef __cplusplus
#define CQSA_INT_ENUM(tag) enum tag : int
#else
#define CQSA_INT_ENUM(tag) enum tag
#endif

typedef CQSA_INT_ENUM(cqsa_status_e) {
  CQSA_OK = 0,
  CQSA_EINVAL = -1,   /* bad argument (null pointer, size, unsupported d/dtype/flag) */
  CQSA_ENOSET = -2,   /* no perfect difference set for this l (l = 7) */
  CQSA_EDIVIDE = -3,  /* N is not a multiple of prod(c_k) (and CQSA_FLAG_PAD unset) or N < prod(c_k) */
  CQSA_EBUDGET = -4,  /* no staging mode fits the memory budget, or a device-resident call's
                         workspace and descriptor tables exceed it */
  CQSA_EHIP = -5,     /* a HIP runtime call failed */
  CQSA_ENOMEM = -6,   /* a host or device allocation failed */
  CQSA_ESMALL = -7    /* a caller buffer or workspace is smaller than required */
} cqsa_status;

typedef CQSA_INT_ENUM(cqsa_dtype_e) { CQSA_BF16 = 0, CQSA_F32 = 1 } cqsa_dtype;

/* Where q, k, v, o and lse live for cqsa_forward. */
typedef CQSA_INT_ENUM(cqsa_residency_e) { CQSA_RES_DEVICE = 0, CQSA_RES_HOST_PINNED = 1 } cqsa_residency;

/* Staging mode of the host-pinned path, chosen by the footprint model. */
typedef CQSA_INT_ENUM(cqsa_mode_e) {
  CQSA_MODE_DEVICE_ACC_KV2 = 1, /* K/V of two tasks staged (double buffer), accumulator on device */
  CQSA_MODE_HOST_ACC_KV2 = 2,   /* K/V double buffer, accumulator in pinned host memory */
  CQSA_MODE_DEVICE_ACC_KV1 = 3, /* one task's K/V resident at a time, accumulator on device */
  CQSA_MODE_HOST_ACC_KV1 = 4    /* one task's K/V resident at a time, accumulator on host */
} cqsa_mode;

/* plan_create flags (all optional; 0 = let the footprint model choose). */
#define CQSA_FLAG_HOST_ACC 0x1u  /* only consider modes with the accumulator on the host */
#define CQSA_FLAG_KV_SINGLE 0x2u /* only consider single-buffered K/V staging */
/* Accept any N: the division runs over N_pad = ceil(N / prod(c_k)) * prod(c_k) tokens and
 * positions >= N are padding that no query block, key run or copy touches, so the result
 * is attention over the N real tokens.  Without this flag an N off the unit grid is EDIVIDE. */
#define CQSA_FLAG_PAD 0x4u
/* Causal attention: row i attends keys j <= i.  The division and owners are unchanged;
 * inside a task (its tokens in ascending order) a unit pair is kept only when the key
 * unit does not come after the query unit, and the diagonal unit block is masked
 * element by element.  useful_flop becomes 2 N (N+1) d H. */
#define CQSA_FLAG_CAUSAL 0x8u
/* Budget from the device: the plan's budget becomes the free memory of the current HIP
 * device (hipMemGetInfo, read once at plan creation) minus budget_bytes, which is then a
 * safety margin (>= 0).  "Stream-CQSA: Exact Out-of-Memory Recovery for Attention",
 * abstract: the attention call is partitioned into subproblems that fit the memory the
 * device has; the Lattice summary: subproblems fit arbitrary memory budgets.  This is
 * the one plan_create option that makes a HIP call; EHIP without a usable device,
 * EBUDGET if the margin exceeds the free memory. */
#define CQSA_FLAG_FREE_BUDGET 0x10u

#define CQSA_MAX_LEVELS 12
#define CQSA_MAX_L 10

typedef struct cqsa_plan cqsa_plan; /* opaque; immutable once created */

typedef struct {
  int64_t n_tokens;
  int32_t heads, head_dim, dtype;
  int32_t levels;               /* itr: number of CQS Divide levels */
  int32_t c[CQSA_MAX_LEVELS];   /* chunks per level, c = l(l-1)+1 */
  int32_t l[CQSA_MAX_LEVELS];   /* chunks per subsequence per level */
  int64_t n_tasks;              /* prod(c_k) innermost tasks */
  int64_t unit_tokens;          /* N / prod(c_k): the ownership grid */
  int64_t n_units;              /* prod(c_k) */
  int64_t visits;               /* prod(l_k): tasks that visit each query row */
  int64_t task_tokens;          /* tokens per innermost task */
  int64_t budget_bytes;         /* 0 = unlimited */
  int32_t stream_mode;          /* cqsa_mode chosen for CQSA_RES_HOST_PINNED */
  int32_t kv_buffers;           /* 1 or 2 */
  int64_t stream_workspace_bytes; /* device bytes the host-pinned path needs (<= budget) */
  int64_t device_workspace_bytes; /* device bytes the device-resident path needs */
  int64_t host_acc_bytes;       /* pinned host accumulator the host-pinned path allocates (0 if on device) */
  double useful_flop;           /* 4 * N^2 * d * H; 2 * N * (N+1) * d * H with CQSA_FLAG_CAUSAL */
  int64_t padded_tokens;        /* N_pad = unit_tokens * n_units (== n_tokens unless padded) */
  int32_t bwd_stream_mode;      /* cqsa_mode of the host-pinned backward, 0 if none fits the budget */
  int32_t bwd_host_stats;       /* 1: that backward keeps L and Delta of every row in pinned host
                                   memory and gathers each task's rows with its staging (chosen
                                   only when no layout with them on the device fits) */
  int64_t bwd_stream_workspace_bytes; /* device bytes of that backward, -1 if none fits */
} cqsa_plan_info;

typedef struct {
  double t_total_ms;            /* wall time of the call (host clock) */
  /* Busy time of each phase: the union of its event-timed intervals over every stream
   * that runs it (copies on two streams at once count once), so bytes / time is the
   * phase's rate while it is active. */
  double t_h2d_ms, t_attn_ms, t_merge_ms, t_d2h_ms;
  int64_t bytes_h2d, bytes_d2h;
  int64_t peak_device_bytes;    /* modelled: workspace + descriptor tables of the plan run */
  int64_t n_attn_launches, n_merge_launches, n_h2d_copies, n_d2h_copies;
  double useful_flop;
  int64_t bytes_d2d;            /* K/V rows reused from the previous task's staging buffer */
  /* Observed: free device memory (hipMemGetInfo) at entry minus its minimum, polled after
   * every allocation and after each task is enqueued.  Device memory the library or the
   * caller held before the call (a caller workspace, descriptor tables an earlier call on
   * the plan uploaded) is not in it. */
  int64_t observed_peak_bytes;
  int64_t device_free_at_entry; /* hipMemGetInfo free bytes when the call began */
  int32_t levels_used;          /* levels of the plan that ran (more than the caller's after a re-plan) */
  int32_t replans;              /* out-of-memory re-plans made inside the call (host-pinned path) */
} cqsa_stats;

/* Measured rates a dry run prices a plan with (all > 0). */
typedef struct {
  double attn_tflops;           /* partial kernel, useful TFLOP/s */
  double merge_gbs;             /* merge kernel, HBM GB/s */
  double h2d_gbs, d2h_gbs;      /* pinned host <-> device copies, GB/s */
} cqsa_rates;

/* Plan-only summary of a (possibly huge) CQS plan: what cqsa_forward with
 * CQSA_RES_HOST_PINNED would stage, move and compute, and the time those rates give. */
typedef struct {
  int64_t n_tokens, padded_tokens;
  int32_t heads, head_dim, dtype;
  int32_t levels;
  int32_t c[CQSA_MAX_LEVELS], l[CQSA_MAX_LEVELS];
  int64_t n_tasks;              /* prod(c_k) */
  int64_t unit_tokens;          /* padded_tokens / prod(c_k) */
  int64_t visits;               /* prod(l_k) */
  int64_t task_tokens;          /* unit_tokens * visits */
  int32_t stream_mode;          /* cqsa_mode that fits the budget, 0 if none */
  int32_t kv_buffers;
  int64_t stream_workspace_bytes; /* device bytes of that mode (excluding descriptor tables) */
  int64_t per_task_descriptor_bytes; /* upper bound of one task's work items + key runs */
  int64_t host_pinned_bytes;    /* Q, K, V, O, LSE in pinned memory + the host accumulator */
  int64_t bytes_h2d, bytes_d2h; /* what the stream engine copies (LSE included); exact for
                                   plans without padding, else bytes_h2d is a lower bound
                                   and bytes_h2d + bytes_d2d is exact */
  int64_t bytes_d2d;            /* K/V rows of shared chunks copied device to device */
  int64_t merge_bytes;          /* HBM bytes of all merge launches */
  double useful_flop;           /* 4 N^2 d H; 2 N (N+1) d H with CQSA_FLAG_CAUSAL */
  double t_attn_s, t_merge_s, t_h2d_s, t_d2h_s;
  double t_est_s;               /* max(attn + merge (+ unoverlapped K/V loads), h2d, d2h) */
  int32_t materializable;       /* 1 if cqsa_plan_create builds this plan */
  /* The host-pinned backward (cqsa_backward) under the same budget: the levels it needs
   * (these levels, or with n_levels = 0 the innermost l repeated further until one of its
   * layouts fits; 0 if none does), its staging mode, whether it keeps L and Delta in
   * pinned host memory, its task size and its device workspace (-1 if none fits). */
  int32_t bwd_levels;
  int32_t bwd_stream_mode;
  int32_t bwd_host_stats;
  int32_t bwd_reserved;         /* 0 */
  int64_t bwd_task_tokens;
  int64_t bwd_stream_workspace_bytes;
} cqsa_estimate;

/* Library version string. */
const char* cqsa_version(void);

/*
 * Perfect difference set of size l (the cyclic quorum behind CQS Divide; "Stream-CQSA:
 * Exact Out-of-Memory Recovery for Attention", abstract: the division rests on cyclic
 * quorum sets).  Writes the lexicographically smallest sorted set D of l
 * residues mod c = l(l-1)+1 with {0,1} in D whose nonzero differences cover 1..c-1
 * exactly once (l = 1 gives {0}).  out: host array of >= l int32 (cap = its length).
 * Errors: EINVAL (l outside 1..CQSA_MAX_L, out NULL, cap < l), ENOSET (l = 7).
 */
cqsa_status cqsa_difference_set(int32_t l, int32_t* out, int32_t cap);

/*
 * Build the CQS plan for an N-token attention ("The 'CQS Divide'" and "The Recursive
 * Benefit" sections of the wispaper explainer; the Lattice summary's memory budget).
 *   l_levels[0..n_levels): l per level, outer level first.  n_levels = 0 means
 *     "auto" (out-of-memory recovery): the undivided plan (l = 1) if the host-pinned
 *     path fits budget_bytes, else l_levels[0] (one value read, 2..10) repeated over
 *     the fewest levels that fit (at most CQSA_MAX_LEVELS); EBUDGET if none does.
 *   Task t (mixed radix over levels, outer first) holds the chunks
 *     sorted{(t_k + d) mod c_k : d in D_k} of its parent at each level; inside a task,
 *     query unit i and key unit j are admitted iff at every level they lie in
 *     different chunks or both in chunk t_k (the CQS Mask: one owner per pair).
 *   budget_bytes: device-memory budget of the host-pinned path (0 = unlimited); the
 *     footprint model picks the first fitting mode in the order of cqsa_mode.
 *   flags: CQSA_FLAG_* above.
 * Host-only (no HIP call).  *out receives a plan owned by the caller (free with
 * cqsa_plan_destroy) or NULL on error.  Errors: EINVAL, ENOSET, EDIVIDE (N off the unit
 * grid without CQSA_FLAG_PAD, or N < prod(c_k)), EBUDGET.
 * Supported: dtype BF16 with head_dim 64 or 128, dtype F32 with head_dim 64 or 128.
 */
cqsa_status cqsa_plan_create(int64_t n, int32_t heads, int32_t head_dim, cqsa_dtype dtype,
                             const int32_t* l_levels, int32_t n_levels, int64_t budget_bytes,
                             uint32_t flags, cqsa_plan** out);

/* Copy the plan's summary into *out (host). Errors: EINVAL. */
cqsa_status cqsa_plan_info_get(const cqsa_plan* plan, cqsa_plan_info* out);

/*
 * Canonical schedule record (int64, host): the tasks of the CQS Divide in the order they
 * run ("The 'CQS Divide'" and "Implementation: From High-Level Logic to GPU Kernels"
 * sections of the wispaper explainer: subsequence tasks, each a set of chunks, with the
 * CQS Mask deciding which key ranges each query range of a task computes).  Layout:
 *   n_levels, (c_k, l_k) per level, n_tasks, unit_tokens, n_units, then per task in
 *   ascending id: tid, t_1..t_L, n_segments, (global_start, length, local_offset) per
 *   segment in tokens, n_query_units, and per local query unit: global_unit, n_runs,
 *   (key_local_unit_start, key_unit_count) per run.
 * Size query: cap = 0 (buf may be NULL) sets *needed.  Errors: EINVAL, ESMALL.
 */
cqsa_status cqsa_plan_schedule(const cqsa_plan* plan, int64_t* buf, int64_t cap, int64_t* needed);

/*
 * Coverage table: int32 [U][U], entry [p][q] = id of the task that owns the pair
 * (query unit p, key unit q).  Each pair has exactly one owner (the Steiner system
 * S(2,l,c) of the "CQS Divide" section).  Size query with cap = 0.  Errors: EINVAL, ESMALL.
 */
cqsa_status cqsa_plan_coverage(const cqsa_plan* plan, int32_t* table, int64_t cap, int64_t* needed);

/* Free a plan, the device descriptor tables it cached and the pinned host accumulator it
 * keeps between streamed forward calls.  NULL is ignored.  No call may be running on it. */
void cqsa_plan_destroy(cqsa_plan* plan);

/*
 * Device workspace the call needs for residency res (bytes).  Pass a buffer of at
 * least this size to cqsa_forward to keep the call free of device allocation.
 */
cqsa_status cqsa_workspace_size(const cqsa_plan* plan, cqsa_residency res, int64_t* bytes);

/*
 * Masked attention partials of every task, device-resident ("Implementation" section
 * of the wispaper explainer: per-task softmax numerator and denominator sums; the CQS
 * Mask selects the keys).  For every task t and every query row i of t:
 *     s_ij = (1/sqrt(d)) <q_i, k_j> over the keys j that t admits for i,
 *     m = a reference with  M - 8 <= m <= M,  M = log2(e) * max_j s_ij
 *         (bf16: moved lazily, so it can trail the max by up to 8; float32: m = M),
 *     l = sum_j 2^(log2(e) s_ij - m),
 *     n = sum_j 2^(log2(e) s_ij - m) v_j            (unnormalised, float32)
 * The triple is exact for whatever m it carries; only m + log2 l and n / l are
 * invariants, and the merge uses nothing else.  A row no key reaches holds
 * (m, l, n) = (-inf, 0, 0).
 * q, k, v: device [N, H, d] in the plan's dtype (read only).
 * n_out: device float32 [V][N][H][d]; ml_out: device float32 [V][N][H][2] holding (m, l);
 *   V = visits; slot s of row i holds the s-th task (ascending id) that visits row i.
 * Enqueued on stream; returns before the kernels finish.  The plan uploads its
 * descriptor table to the device once (kept until cqsa_plan_destroy).
 * Errors: EINVAL, EHIP, ENOMEM.
 */
cqsa_status cqsa_partials(const cqsa_plan* plan, const void* q, const void* k, const void* v,
                          float* n_out, float* ml_out, void* stream);

/*
 * Recompose partials into the output ("recomposes the local statistics", abstract of
 * arXiv 2604.20819).  Folds the V slots of each (row, head) in ascending slot order:
 *     m = max(m_a, m_b), l = l_a 2^(m_a-m) + l_b 2^(m_b-m), n likewise,
 * then O = n / l in the plan's dtype (round to nearest even for bf16) and
 * LSE = ln(2) * (m + log2 l).
 * n_in, ml_in: device, layout of cqsa_partials.  o: device [N, H, d] dtype.
 * lse: device float32 [H, N] or NULL.  Enqueued on stream.  Errors: EINVAL, EHIP.
 */
cqsa_status cqsa_merge(const cqsa_plan* plan, const float* n_in, const float* ml_in,
                       void* o, float* lse, void* stream);

/*
 * Full CQS forward: O = softmax(Q K^T / sqrt(d)) V and LSE, exact up to rounding (with
 * CQSA_FLAG_CAUSAL the softmax runs over keys j <= i).  "Stream-CQSA: Exact
 * Out-of-Memory Recovery for Attention", abstract: independent subsequence tasks whose
 * local statistics recompose into the full output; "Stream-CQSA: Breaking the
 * Billion-Token Barrier on a Single GPU", section "Implementation: From High-Level Logic
 * to GPU Kernels": each task's Q, K, V moved to the device, per-task softmax sums,
 * aggregation in host memory; Lattice summary: subproblems within a memory budget.
 *   CQSA_RES_DEVICE: q, k, v, o, lse are device pointers; runs cqsa_partials then
 *     cqsa_merge on stream using `workspace` (>= cqsa_workspace_size bytes) for the
 *     partial slots.  Stream-ordered: returns after enqueuing unless the library had
 *     to allocate the workspace itself (workspace == NULL), or stats != NULL.
 *   CQSA_RES_HOST_PINNED: q, k, v, o, lse are pinned host pointers (lse may be NULL);
 *     a device pointer or pageable host memory among them is EINVAL, before any copy.
 *     Tasks run in ascending id; each task's K/V segments are gathered into device
 *     staging with hipMemcpyAsync on copy streams, double-buffered when the mode says
 *     so, query units are streamed in blocks, partials are merged into the
 *     accumulator (device, or pinned host memory with H2D/D2H round trips: allocated by
 *     the plan's first such call, N*H*(d+2)*4 bytes, and kept with the plan until
 *     cqsa_plan_destroy; a call made while another uses it allocates its own), and the
 *     finished O blocks are copied back as each unit completes; LSE is kept [H][N] on
 *     the device for the call and copied back once at the end when that takes at most
 *     1/16 of the budget (always without one), else copied back per unit block, one
 *     copy per head.  Device memory used is
 *     the workspace (<= budget).  Synchronous: returns after all work is complete.  If
 *     the library must allocate the workspace and the device is out of memory, the
 *     call re-plans one level deeper (cqsa_plan_fallback, budget = free memory minus
 *     1/16) and retries, up to CQSA_MAX_LEVELS levels; the caller's plan is unchanged.
 * workspace: device buffer or NULL (then the library allocates exactly the size
 *   needed and frees it before returning).  lse may be NULL.
 * stats: optional; when given, phases are timed with HIP events.
 * Debugging aids (environment, read at each call): CQSA_SYNC=1 waits for the device
 *   after every step the host-pinned path enqueues (streams effectively serialised);
 *   CQSA_CANARY=1 surrounds every piece of the host-pinned workspace with guard words
 *   and checks them after the call (EHIP naming the piece if one was overwritten).
 * Errors: EINVAL, ESMALL, EBUDGET (device path: workspace plus descriptor tables over the budget), EHIP, ENOMEM.
 */
cqsa_status cqsa_forward(const cqsa_plan* plan, const void* q, const void* k, const void* v,
                         void* o, float* lse, cqsa_residency res, void* workspace,
                         int64_t workspace_bytes, void* stream, cqsa_stats* stats);

/*
 * cqsa_forward with CQSA_RES_DEVICE for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and the same result, bit for bit, but the partial slots and the forward
 * descriptor tables live in a fixed array of device memory of the library, 256 MiB on
 * each device the library runs on, held from this call's first use on the device until
 * the process ends.  The plan must need at most that much:
 *     align256(V*N*H*d*4) + align256(V*N*H*2*4) + align256(items*32) + align256(runs*16)
 *     (+ align256(4 * blocks) for a causal plan's dispatch order of the launch)
 * (V = visits; e.g. N = 14,336, H = 8, d = 128 with one level of l = 3 needs 179 MB);
 * a larger plan gets ESMALL and nothing is enqueued.  Nothing is allocated or freed, and
 * the plan's own device tables are not used: each call copies the forward descriptor
 * table from the plan's host memory into the array with hipMemcpyAsync on stream.
 * The array keeps what the last call left; nothing in it is read before the call writes
 * it.  Every call on one device shares that device's array: calls that overlap on one
 * device (on different streams, or from several threads) race; calls on one stream are
 * ordered.  The plan's budget is not applied (the array is the bound).
 * q, k, v, o, lse: device pointers, layouts of cqsa_forward (lse may be NULL).
 * Enqueued on stream; returns before the kernels finish.
 * Errors: EINVAL (NULL or misaligned pointer), ESMALL (plan larger than the array), EHIP.
 */
cqsa_status cqsa_forward_noalloc(const cqsa_plan* plan, const void* q, const void* k, const void* v,
                                 void* o, float* lse, void* stream);

/*
 * Device workspace bytes cqsa_backward needs for res.  CQSA_RES_DEVICE: Delta [H][N]
 * fp32, for bf16 three transposed copies (Q, K, dO) [H][d][round_up(N, 64)], and the
 * visit slots of dQ, dK, dV [V][N][H][d] fp32 (V = prod(l_k)).  CQSA_RES_HOST_PINNED:
 * L and Delta [H][N]; one task's Q, K, V, dO and their transposes; the task's L and
 * Delta rows; a two-slot ring of unit blocks (terms, output, and host-accumulator
 * blocks); fp32 accumulators [N][H][d] for dQ, dK, dV when they fit the plan's budget
 * (else they live in pinned host memory and are not counted).
 * Errors: EINVAL (NULL or unknown residency), EBUDGET (no streamed layout fits).
 */
cqsa_status cqsa_backward_workspace_size(const cqsa_plan* plan, cqsa_residency res, int64_t* bytes);

/*
 * Backward of the CQS forward: gradients of O = softmax(Q K^T / sqrt(d)) V for an
 * upstream gradient dO ("Stream-CQSA: Exact Out-of-Memory Recovery for Attention",
 * abstract: the decomposition is exact for the backward pass as well).  With the
 * forward's final LSE every admitted (query, key) pair contributes independently:
 *     P = exp(s - LSE), Delta_i = <dO_i, O_i>, dS = P (dO_i.v_j - Delta_i),
 *     dV_j += P dO_i, dK_j += dS q_i / sqrt(d), dQ_i += dS k_j / sqrt(d),
 * and the CQS Mask gives each pair to exactly one task, so each task's terms go to
 * the rows' visit slots and the slots are summed in ascending task order
 * (deterministic; no rescaling across tasks).
 *   q, k, v, o, d_o: [N, H, d] in the plan's dtype (read only); o and lse are the
 *     forward's outputs (lse: float32 [H, N], natural log).
 *   dq, dk, dv: [N, H, d] in the plan's dtype (written; round to nearest even).
 *   res: CQSA_RES_DEVICE (device pointers; stream-ordered like cqsa_forward) or
 *     CQSA_RES_HOST_PINNED (pinned host pointers, else EINVAL before any copy;
 *     synchronous): Delta of every row is
 *     formed first from O and dO streamed in unit blocks; then per task in ascending id
 *     its Q, K, V, dO rows are staged and transposed on the device, its L and Delta
 *     rows gathered, and for each of its units the dQ and dK/dV terms are added into
 *     the unit's accumulators (device, or pinned host memory with round trips) in the
 *     device path's order, so both residencies give the same bits.  Device memory used
 *     is the workspace (<= the plan's budget).
 *   workspace: device buffer >= cqsa_backward_workspace_size(res) bytes, or NULL (the
 *     library allocates and frees it).
 *   stats: optional; t_attn_ms = the two gradient kernels, t_merge_ms = the Delta /
 *     transpose pass and the slot sums, useful_flop = 2.5 times the forward's
 *     (10 N^2 d H; 5 N (N+1) d H with CQSA_FLAG_CAUSAL).
 * Errors: EINVAL, ESMALL, EBUDGET (workspace plus the plan's descriptor tables over its budget), EHIP, ENOMEM.
 */
cqsa_status cqsa_backward(const cqsa_plan* plan, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                          void* dv, cqsa_residency res, void* workspace, int64_t workspace_bytes,
                          void* stream, cqsa_stats* stats);

/*
 * Dry run of the streamed forward for any N ("The Recursive Benefit" and "Precise
 * Scaling" sections of the wispaper explainer: recursion depth for very long
 * sequences): the same levels, footprint model, budget test and mode choice as
 * cqsa_plan_create (n_levels = 0: undivided first, then l_levels[0] repeated, up to
 * CQSA_MAX_LEVELS), in closed form.  The budget test is cqsa_plan_create's: workspace
 * plus descriptor tables.  For a plan cqsa_plan_create would build, the tables are
 * built here (host time and memory grow with tasks x units^2: seconds for millions of
 * items) when a shape bound cannot settle the test; a plan too large to build is
 * estimated without them (they would have to be streamed per task;
 * per_task_descriptor_bytes bounds one task's share), so itr up to CQSA_MAX_LEVELS and
 * billions of tokens stay cheap.  Bytes and FLOP are exact for the stream engine (with
 * LSE returned); times come from `rates` (measured by the caller), overlapping copies
 * with compute as the engine does (a single-buffered K/V stage is not overlapped).
 * stream_workspace_bytes excludes the descriptor tables.
 * Host-only.  Errors: EINVAL, ENOSET, EDIVIDE, EBUDGET (no mode fits at any depth).
 */
cqsa_status cqsa_plan_estimate(int64_t n, int32_t heads, int32_t head_dim, cqsa_dtype dtype,
                               const int32_t* l_levels, int32_t n_levels, int64_t budget_bytes,
                               uint32_t flags, const cqsa_rates* rates, cqsa_estimate* out);

/*
 * The plan the out-of-memory recovery falls back to: one CQS Divide level deeper than
 * `plan` ("Stream-CQSA: Exact Out-of-Memory Recovery for Attention", abstract: a
 * memory-capacity failure becomes a recoverable execution path; "The Recursive Benefit"
 * section of the wispaper explainer: a task that is still too large is divided again).
 * The new level repeats the l of the plan's innermost level (3 if that l is 1, an
 * undivided plan); CQSA_FLAG_PAD is added when N no longer divides into the deeper unit
 * grid (exact: padding is never read).  budget_bytes (> 0) replaces the plan's budget;
 * if even the deeper plan's footprint exceeds it, further levels are added until one
 * fits.  Every other property (dtype, causality, flags) is kept.  When the host-pinned
 * cqsa_forward cannot allocate its device workspace (ENOMEM from the HIP allocator and
 * no caller workspace), it builds this plan with the device's free memory minus 1/16 as
 * the budget and runs it inside the same call (stats.replans counts such re-plans).
 * Host-only.  *out receives a plan the caller frees with cqsa_plan_destroy.  Errors:
 * EINVAL, EBUDGET (no depth up to CQSA_MAX_LEVELS fits), EDIVIDE (fewer tokens than
 * units), ENOMEM (the deeper plan is too large to build).
 */
cqsa_status cqsa_plan_fallback(const cqsa_plan* plan, int64_t budget_bytes, cqsa_plan** out);

/*
 * Fault injection for tests of the recovery paths (callers: test suites only).  The
 * next `count` device allocations the library makes (workspaces, descriptor tables)
 * fail as if the device were out of memory, without calling the HIP allocator; 0
 * clears it.  Process-wide.  Errors: EINVAL (count < 0).
 */
cqsa_status cqsa_debug_fail_allocations(int32_t count);

/* Static text for a status code. */
const char* cqsa_status_string(cqsa_status status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* cqsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CQSA_H */
