// HIP kernels for gfx950 (MI355X, CDNA4): masked attention partials and the merge of
// (max, denominator, numerator) statistics.
//
// What they compute follows "Stream-CQSA: Breaking the Billion-Token Barrier on a
// Single GPU" (wispaper explainer), section "Implementation: From High-Level Logic to
// GPU Kernels" (each task's softmax numerator and denominator sums, the CQS Mask
// selecting the keys) and the abstract of arXiv 2604.20819 (recompose the local
// statistics).  The running-max form of the partials is the online normaliser of
// "Online normalizer calculation for softmax" (cited by title on the arXiv page).
//
// Partial of one task for query row i:   (log2 units throughout)
//   m = a reference at most 8 below log2(e) * max_j s_ij (the bf16 kernel moves it
//       lazily; the fp32 kernel keeps the running max),
//   l = sum_j 2^(log2(e) s_ij - m),  n = sum_j 2^(log2(e) s_ij - m) v_j
// over the keys admitted for i; (m, l, n) is exact for whatever m it carries.  The kernel design (tiles, LDS layout, MFMA shapes) is
// this library's own for CDNA4 wave64 hardware.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace cqsa {

namespace {

using namespace dev;


struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  float* n_out;
  float* ml_out;
  const WorkItem* items;
  const KeyRun* runs;
  const int32_t* order;  // dispatch order, or null
  int64_t n_items;
  int tiles_per_item;
  int heads;
  float scale_log2;
};

// The (item, head, tile) this workgroup computes: from the planner's dispatch order when
// the launch has one (block b runs entry b; -1 marks a block with nothing to do), else
// the arithmetic order of group_coord.
__device__ __forceinline__ bool attn_coord(const AttnParams& P, GroupCoord& c) {
  if (P.order == nullptr) return group_coord(blockIdx.x, P.tiles_per_item, P.heads, P.n_items, c);
  const int v = P.order[blockIdx.x];
  if (v < 0) return false;
  c.tile = v % P.tiles_per_item;
  const int g = v / P.tiles_per_item;
  c.head = g % P.heads;
  c.item = g / P.heads;
  return true;
}


// ---------------------------------------------------------------------------------
// bf16 partials on MFMA.  Workgroup = 8 wave64 = 256 query rows (32 per wave); all
// eight waves share each 64-key K/V tile, so a tile fetched from L2 feeds 256 queries.
//
// S^T (keys x queries) = K_tile * Q^T with v_mfma_f32_32x32x16_bf16: A = 32 key rows
// read from LDS, B = this lane's query slice held in registers.  Each lane then owns
// one query column and 16 key rows of every 32x32 score tile, so the softmax row
// statistics are lane-local plus one exchange with lane^32.  The K rows of an MFMA
// tile are read in an order that swaps bits 2 and 3 of the row index; with that order
// the 16 accumulator values a lane holds are exactly the B operand (8 consecutive
// keys per half-wave) of O^T += V^T * P^T, so P never leaves registers.  V stays
// row-major in LDS and the A operand of that product (8 consecutive keys of one dim
// per lane) is fetched with two LDS transpose reads (ds_read_b64_tr_b16).
//
// Pipeline: the next tile is fetched from global memory into registers while the
// current one is computed from LDS, then written to the other LDS stage; one barrier
// per tile.  The running max is a lazily moved reference: the weights of a tile are
// formed against it first, and it moves (with a rescale of l and n and a recompute of
// the weights) only when a lane's weights sum to more than 2^8 or to a non-finite
// value.  Every weight therefore stays <= 2^8, the triple (m, l, n) remains exact for
// whatever m it carries, and the common path needs no max over the tile.
// ---------------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr float kLazySum = 256.0f;  // largest row sum of a lane's weights kept without moving m

template <int D>
struct Bf16Tile {
  static constexpr int NW = 8;          // waves per workgroup
  static constexpr int NT = 64 * NW;    // threads
  static constexpr int QT = 32 * NW;    // query rows per workgroup
  static constexpr int KT = 64;         // keys per tile
  static constexpr int KSTR = D + 8;    // K row stride in LDS (u16): 16-byte pad
  static constexpr int VSTR = D + 32;   // V row stride in LDS (u16): rows 16 dwords apart mod 64 banks
  static constexpr int DCH = D / 8;     // 16-byte chunks per row
  static constexpr int CPT = KT * DCH / NT;  // chunks of K (and of V) per thread per tile
  static constexpr int KBYTES = KT * KSTR * 2;
  static constexpr int VBYTES = KT * VSTR * 2;
  static constexpr int STAGE = KBYTES + VBYTES;
  static_assert(CPT >= 1 && KT * DCH == CPT * NT, "tile split");
};


template <int D>
__global__ __launch_bounds__(512) void attn_partial_bf16(AttnParams P) {
  using T = Bf16Tile<D>;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  GroupCoord gc;
  if (!attn_coord(P, gc)) return;
  const int tile = gc.tile;
  const int head = gc.head;
  const WorkItem it = P.items[gc.item];
  const KeyRun* runs = P.runs + it.run0;
  const int nrun = it.nrun;
  const int64_t rs = static_cast<int64_t>(P.heads) * D;
  const u16* __restrict__ Q = static_cast<const u16*>(P.q);
  const u16* __restrict__ K = static_cast<const u16*>(P.k) + head * D;
  const u16* __restrict__ V = static_cast<const u16*>(P.v) + head * D;

  const int qi = tile * T::QT + wave * 32 + col;
  const bool qok = qi < it.q_len;
  bf16x8 qf[NKK];
  {
    const u16* qp = Q + (it.q_row0 + (qok ? qi : 0)) * rs + head * D + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qok) u = *reinterpret_cast<const uint4*>(qp + 16 * kk);
      qf[kk] = as_bf16x8(u);
    }
  }
  // Complete the Q loads here, on every path into the key loop.  Otherwise the wait for
  // them lands on the loop's first score product, inside the loop, where it also waits
  // for the next tile's loads in flight on every iteration.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(qf[kk]));

  // global -> register fetch of one tile.  Each thread's chunks sit at fixed offsets
  // from the tile's first row (computed once); on a run's ragged last tile the rows past
  // the end repeat the run's last row, so no read leaves the run, and their scores are
  // masked to -inf (weight exactly 0).
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 kr[T::CPT], vr[T::CPT];
  const uint32_t fcol = (tid % T::DCH) * 8;
  const uint32_t fbase = static_cast<uint32_t>(tid / T::DCH) * static_cast<uint32_t>(rs) + fcol;
  const uint32_t fstep = static_cast<uint32_t>(T::NT / T::DCH) * static_cast<uint32_t>(rs);
  auto fetch = [&](const TileCursor& c) {
    const u16* kb = K + (c.start + c.k0) * rs;
    const u16* vb = V + (c.start + c.k0) * rs;
    const uint32_t last = static_cast<uint32_t>(min(T::KT, c.len - c.k0) - 1) * static_cast<uint32_t>(rs) + fcol;
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const uint32_t o = fbase + i * fstep;
      const uint32_t off = o < last ? o : last;
      kr[i] = *reinterpret_cast<const u32x4*>(kb + off);
      vr[i] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  };
  auto stash = [&](int stage) {
    u16* ks = reinterpret_cast<u16*>(smem + stage * T::STAGE);
    u16* vs = reinterpret_cast<u16*>(smem + stage * T::STAGE + T::KBYTES);
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int ch = tid + i * T::NT;
      const int row = ch / T::DCH, cc = ch % T::DCH;
      *reinterpret_cast<u32x4*>(ks + row * T::KSTR + cc * 8) = kr[i];
      *reinterpret_cast<u32x4*>(vs + row * T::VSTR + cc * 8) = vr[i];
    }
  };

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = P.scale_log2;
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  const int prow = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
  // LDS transpose-read address of this lane inside a 4-key x 16-dim block
  const int grp = lane >> 4, sl = lane & 15;
  const int tr_off = (8 * (grp >> 1) + (sl >> 2)) * T::VSTR + 16 * (grp & 1) + 4 * (sl & 3);

  // queries of this workgroup: [tile * QT, qhi) of the item
  const int qhi = min(it.q_len, (tile + 1) * T::QT);
  TileCursor cur = cursor_begin(runs, nrun, qhi);
  TileCursor nxt = cur;
  int stage = 0;
  if (cur.run < nrun) {
    fetch(cur);
    stash(0);
    cursor_next(nxt, runs, nrun, T::KT, qhi);
    if (nxt.run < nrun) fetch(nxt);
  }
  __syncthreads();

  while (cur.run < nrun) {
    // Scheduling hint: the backend's MFMA/LDS interleaving for a single wave's tile loop
    // (measured 1.8 % faster here, identical bits).
    __builtin_amdgcn_iglp_opt(1);
    const int nv = min(T::KT, cur.len - cur.k0);
    const u16* ks = reinterpret_cast<const u16*>(smem + stage * T::STAGE);
    const u16* vs = reinterpret_cast<const u16*>(smem + stage * T::STAGE + T::KBYTES);

    // scores S^T for keys [0,32) and [32,64)
    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
    {
      const u16* kp = ks + prow * T::KSTR + 8 * hl;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(kp + 32 * st * T::KSTR + 16 * kk));
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[st], 0, 0, 0);
        }
    }
    // accumulator element i of tile st holds key 32*st + 16*(i/8) + 8*hl + i%8
    if (nv < T::KT) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * st + 16 * (i >> 3) + 8 * hl + (i & 7) >= nv) s[st][i] = -INFINITY;
    }
    // causal diagonal: this lane's query qi sees key k0 + j only if k0 + j <= diag + qi
    if (cur.diag >= 0 && cur.k0 + T::KT - 1 > cur.diag + tile * T::QT) {
      const int lim = cur.diag + qi - cur.k0;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * st + 16 * (i >> 3) + 8 * hl + (i & 7) > lim) s[st][i] = -INFINITY;
    }
    // Weights against the current reference m, and their row sum over the bf16-rounded
    // values (the same values the P V product uses).  The weights are non-negative, so a
    // lane whose sum is <= 2^8 has every weight <= 2^8.  A larger or non-finite sum (a
    // row's first tile meets m = -inf) sends the wave to the rare branch: m moves to the
    // tile max (both half-waves), l and O are rescaled, and the weights are recomputed.
    bf16x8 pf[4];
    float ps0 = 0.f, ps1 = 0.f;
    auto weights = [&]() {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pf[2 * st + (i >> 3)][i & 7] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[st][i], c2, -m_run)));
      ps0 = 0.f;
      ps1 = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[q], pf[q], 0, 1), ones, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[q], pf[q], 2, 3), ones, ps1, false);
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[q], pf[q], 4, 5), ones, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[q], pf[q], 6, 7), ones, ps1, false);
      }
    };
    weights();
    if (__any(!(ps0 + ps1 <= kLazySum))) {
      float mx = s[0][0];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[st][i]);
      mx *= c2;
      const float m_new = fmaxf(m_run, fmaxf(mx, __shfl_xor(mx, 32)));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      m_run = m_new;
      weights();
    }
    l_run += ps0 + ps1;
    // O^T (dims x queries) += V^T * P^T, 16 keys per step
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int kp4 = 0; kp4 < 4; ++kp4) {
        const u16* vp = vs + tr_off + 16 * kp4 * T::VSTR + 32 * dt;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 4 * T::VSTR));
        const v4i16 both[2] = {lo, hi};
        const bf16x8 a = __builtin_bit_cast(bf16x8, both);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kp4], o[dt], 0, 0, 0);
      }
    }

    // advance: stash the prefetched tile into the other stage, prefetch the one after
    cur = nxt;
    if (cur.run < nrun) {
      stash(stage ^ 1);
      cursor_next(nxt, runs, nrun, T::KT, qhi);
      if (nxt.run < nrun) fetch(nxt);
    }
    stage ^= 1;
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qok) {
    const int64_t orow = it.out_row0 + qi;
    float* np = P.n_out + (orow * P.heads + head) * D;
    // accumulator element i of tile dt holds dim 32*dt + 8*(i/4) + 4*hl + i%4
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 val = make_float4(o[dt][4 * g], o[dt][4 * g + 1], o[dt][4 * g + 2], o[dt][4 * g + 3]);
        *reinterpret_cast<float4*>(np + 32 * dt + 8 * g + 4 * hl) = val;
      }
    if (hl == 0) *reinterpret_cast<float2*>(P.ml_out + (orow * P.heads + head) * 2) = make_float2(m_run, l_tot);
  }
}

// ---------------------------------------------------------------------------------
// float32 partials (correctness path for float32 inputs): one wave of 64 query rows,
// one row per lane, K/V tiles of 32 keys in LDS read by broadcast, fp32 FMA.
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_partial_f32(AttnParams P) {
  constexpr int QT = kAttnQueryTileF32;
  constexpr int KT = kAttnKeyTileF32;
  __shared__ __attribute__((aligned(16))) float kf[KT * D];
  __shared__ __attribute__((aligned(16))) float vf[KT * D];
  const int lane = threadIdx.x;
  GroupCoord gc;
  if (!attn_coord(P, gc)) return;
  const int tile = gc.tile;
  const int head = gc.head;
  const WorkItem it = P.items[gc.item];
  const int64_t rs = static_cast<int64_t>(P.heads) * D;
  const float* __restrict__ Q = static_cast<const float*>(P.q);
  const float* __restrict__ K = static_cast<const float*>(P.k);
  const float* __restrict__ V = static_cast<const float*>(P.v);

  const int qi = tile * QT + lane;
  const bool qok = qi < it.q_len;
  float q[D], o[D];
  {
    const float* qp = Q + (it.q_row0 + (qok ? qi : 0)) * rs + head * D;
#pragma unroll
    for (int t = 0; t < D; t += 4) {
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (qok) u = *reinterpret_cast<const float4*>(qp + t);
      q[t] = u.x;
      q[t + 1] = u.y;
      q[t + 2] = u.z;
      q[t + 3] = u.w;
      o[t] = o[t + 1] = o[t + 2] = o[t + 3] = 0.f;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = P.scale_log2;
  const int qhi = min(it.q_len, (tile + 1) * QT);
  for (int ri = 0; ri < it.nrun; ++ri) {
    const KeyRun run = P.runs[it.run0 + ri];
    const int rlen = run.diag >= 0 ? min(run.len, run.diag + qhi) : run.len;
    // causal diagonal run: key k0 + j is visible to this row only if k0 + j <= lim
    const int lim = run.diag >= 0 ? run.diag + qi : 0x7FFFFFFF;
    for (int k0 = 0; k0 < rlen; k0 += KT) {
      const int nv = min(KT, rlen - k0);
      const int64_t kbase = (run.start + k0) * rs + head * D;
      __syncthreads();
      for (int c = lane; c < KT * D / 4; c += 64) {
        const int kr = c / (D / 4), kc = c % (D / 4);
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (kr < nv) {
          kv = *reinterpret_cast<const float4*>(K + kbase + kr * rs + kc * 4);
          vv = *reinterpret_cast<const float4*>(V + kbase + kr * rs + kc * 4);
        }
        *reinterpret_cast<float4*>(kf + kr * D + kc * 4) = kv;
        *reinterpret_cast<float4*>(vf + kr * D + kc * 4) = vv;
      }
      __syncthreads();
      float sc[KT];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < D; ++t) acc = fmaf(q[t], kf[j * D + t], acc);
        sc[j] = j < nv && k0 + j <= lim ? acc * c2 : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < D; ++t) o[t] *= alpha;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        const float pv = __builtin_amdgcn_exp2f(sc[j] - m_use);
        l_run += pv;
#pragma unroll
        for (int t = 0; t < D; ++t) o[t] = fmaf(pv, vf[j * D + t], o[t]);
      }
      m_run = m_new;
    }
  }
  if (qok) {
    const int64_t orow = it.out_row0 + qi;
    float* np = P.n_out + (orow * P.heads + head) * D;
#pragma unroll
    for (int t = 0; t < D; t += 4) *reinterpret_cast<float4*>(np + t) = make_float4(o[t], o[t + 1], o[t + 2], o[t + 3]);
    *reinterpret_cast<float2*>(P.ml_out + (orow * P.heads + head) * 2) = make_float2(m_run, l_run);
  }
}

// ---------------------------------------------------------------------------------
// Merge: D/4 lanes per (row, head), one float4 of n each; fold inputs in order.
// ---------------------------------------------------------------------------------
struct MergeParams {
  const float* n_a;
  const float* ml_a;
  const float* n_b;
  const float* ml_b;
  int64_t b_stride_n, b_stride_ml;
  int nb;
  int heads;
  int64_t pairs;
  int final_out;
  float* n_out;
  float* ml_out;
  void* o_out;
  float* lse_out;
  int64_t lse_stride, lse_row0;
};


template <int D, typename OutT>
__global__ __launch_bounds__(256) void merge_partials(MergeParams P) {
  constexpr int TPR = D / 4;
  constexpr int PPB = 256 / TPR;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * PPB + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  if (pair >= P.pairs) return;
  const float2 mla = *reinterpret_cast<const float2*>(P.ml_a + 2 * pair);
  float4 n = *reinterpret_cast<const float4*>(P.n_a + pair * D + 4 * t);
  float m = mla.x, l = mla.y;
  for (int s = 0; s < P.nb; ++s) {
    const float2 mlb = *reinterpret_cast<const float2*>(P.ml_b + s * P.b_stride_ml + 2 * pair);
    const float4 nb = *reinterpret_cast<const float4*>(P.n_b + s * P.b_stride_n + pair * D + 4 * t);
    const float mn = fmaxf(m, mlb.x);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float wa = __builtin_amdgcn_exp2f(m - mu);
    const float wb = __builtin_amdgcn_exp2f(mlb.x - mu);
    l = fmaf(l, wa, mlb.y * wb);
    n.x = fmaf(n.x, wa, nb.x * wb);
    n.y = fmaf(n.y, wa, nb.y * wb);
    n.z = fmaf(n.z, wa, nb.z * wb);
    n.w = fmaf(n.w, wa, nb.w * wb);
    m = mn;
  }
  if (!P.final_out) {
    *reinterpret_cast<float4*>(P.n_out + pair * D + 4 * t) = n;
    if (t == 0) *reinterpret_cast<float2*>(P.ml_out + 2 * pair) = make_float2(m, l);
    return;
  }
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
  if (l > 0.f) y = make_float4(n.x / l, n.y / l, n.z / l, n.w / l);
  store_out(static_cast<OutT*>(P.o_out) + pair * D + 4 * t, y);
  if (t == 0 && P.lse_out != nullptr) {
    const int64_t row = pair / P.heads;
    const int head = static_cast<int>(pair % P.heads);
    const float lse = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
    P.lse_out[head * P.lse_stride + P.lse_row0 + row] = lse;
  }
}

}  // namespace

static_assert(Bf16Tile<128>::QT == kAttnQueryTileBf16 && Bf16Tile<64>::QT == kAttnQueryTileBf16 &&
                  Bf16Tile<128>::KT == kAttnKeyTileBf16 && Bf16Tile<64>::KT == kAttnKeyTileBf16,
              "the planner's dispatch order uses the kernel's tile shape");

int attn_query_tile(cqsa_dtype dtype) { return dtype == CQSA_BF16 ? kAttnQueryTileBf16 : kAttnQueryTileF32; }

hipError_t launch_attn(const AttnLaunch& a, hipStream_t stream) {
  if (a.n_items <= 0 || a.q_len <= 0) return hipSuccess;
  AttnParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.n_out = a.n_out;
  p.ml_out = a.ml_out;
  p.items = a.items;
  p.runs = a.runs;
  p.heads = a.heads;
  p.scale_log2 = a.scale_log2;
  p.order = a.order;
  const int qt = attn_query_tile(a.dtype);
  p.tiles_per_item = (a.q_len + qt - 1) / qt;
  p.n_items = a.n_items;
  const int64_t blocks = a.order != nullptr ? a.order_len : group_grid(int64_t(a.n_items) * a.heads, p.tiles_per_item);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a.dtype == CQSA_BF16) {
    if (a.d == 128)
      hipLaunchKernelGGL(attn_partial_bf16<128>, grid, dim3(Bf16Tile<128>::NT), 0, stream, p);
    else if (a.d == 64)
      hipLaunchKernelGGL(attn_partial_bf16<64>, grid, dim3(Bf16Tile<64>::NT), 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL(attn_partial_f32<128>, grid, dim3(64), 0, stream, p);
    else if (a.d == 64)
      hipLaunchKernelGGL(attn_partial_f32<64>, grid, dim3(64), 0, stream, p);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeLaunch& m, hipStream_t stream) {
  if (m.rows <= 0) return hipSuccess;
  MergeParams p;
  p.n_a = m.n_a;
  p.ml_a = m.ml_a;
  p.n_b = m.n_b;
  p.ml_b = m.ml_b;
  p.b_stride_n = m.b_stride_n;
  p.b_stride_ml = m.b_stride_ml;
  p.nb = m.nb;
  p.heads = m.heads;
  p.pairs = m.rows * m.heads;
  p.final_out = m.final_out ? 1 : 0;
  p.n_out = m.n_out;
  p.ml_out = m.ml_out;
  p.o_out = m.o_out;
  p.lse_out = m.lse_out;
  p.lse_stride = m.lse_stride;
  p.lse_row0 = m.lse_row0;
  const int tpr = m.d / 4;
  const int64_t ppb = 256 / tpr;
  const int64_t blocks = (p.pairs + ppb - 1) / ppb;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  const bool bf = m.dtype == CQSA_BF16;
  if (m.d == 128) {
    if (bf)
      hipLaunchKernelGGL((merge_partials<128, u16>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((merge_partials<128, float>), grid, dim3(256), 0, stream, p);
  } else if (m.d == 64) {
    if (bf)
      hipLaunchKernelGGL((merge_partials<64, u16>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((merge_partials<64, float>), grid, dim3(256), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cqsa
