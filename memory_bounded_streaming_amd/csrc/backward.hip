// HIP kernels for gfx950 (MI355X, CDNA4): the backward pass of CQS-divided attention.
//
// "Stream-CQSA: Exact Out-of-Memory Recovery for Attention" (arXiv 2604.20819,
// abstract) states that the decomposition is exact for the backward pass too.  With
// the forward's final log-sum-exp L_i, every admitted (query i, key j) pair contributes
// independently of every other pair (per head, scale c, natural logs):
//
//   P_ij = exp(c q_i.k_j - L_i)          Delta_i = <dO_i, O_i>
//   dS_ij = P_ij (<dO_i, v_j> - Delta_i)
//   dV_j += P_ij dO_i      dK_j += c dS_ij q_i      dQ_i += c dS_ij k_j
//
// and the CQS Mask admits each pair in exactly one task, so the gradient of a row is
// the plain sum of its tasks' terms (no rescaling across tasks).  Every task term is
// written to the row's visit slot (the same slots as the forward partials) and the
// slots are summed in ascending task order, which keeps the result deterministic.
//
// Kernels:
//   bwd_prep            Delta, and (bf16) transposed copies Q^T, K^T, dO^T [H][D][NP]
//   attn_bwd_dkdv_bf16  per (task, key block): dK, dV terms over the admitted query runs
//   attn_bwd_dq_bf16    per (task, query block): dQ terms over the admitted key runs
//   *_f32               the same for float32 inputs with fp32 FMA (correctness path)
//   sum_slots           dX = sum over visit slots, rounded to the input dtype
// The CQS Mask is symmetric (a pair of units is admitted iff at every level the units
// lie in different chunks or both in the task's own chunk), so the admitted query runs
// of a key block are the admitted key runs of the same block as queries: both kernels
// walk the forward's descriptor tables.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace cqsa {

namespace {

using namespace dev;

constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  const u16* qt;       // [H][D][np] (bf16 path)
  const u16* kt;
  const u16* dot;
  const float* lse;    // [H][n], natural log
  const float* delta;  // [H][n]
  float* g0;           // dkdv: dK slots; dq: dQ slots   [slots][n][H][D]
  float* g1;           // dkdv: dV slots
  const WorkItem* items;
  const KeyRun* runs;
  int64_t n_items;
  int64_t n, np;
  int tiles_per_item;
  int heads;
  float scale_log2;    // scale * log2(e)
  float scale;
};

// ---------------------------------------------------------------------------------
// Prep: one workgroup per (64-token tile, head).  Delta = <dO, O> in fp32; for bf16
// inputs also writes Q, K and dO transposed to [H][D][np] (np = n rounded up to 64,
// tokens past n written as zero), so the backward kernels read every operand that is
// contracted over tokens with plain 16-byte LDS reads.
// ---------------------------------------------------------------------------------
struct PrepParams {
  const void* q;
  const void* k;
  const void* o;
  const void* d_o;
  float* delta;         // [H][dpitch], or null: no Delta
  u16* qt;              // null: no transposed copies
  u16* kt;
  u16* dot;
  int64_t n, np, dpitch;
  int heads;
};

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const u16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xFFFF0000u),
                     __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xFFFF0000u));
}

template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_prep(PrepParams P) {
  constexpr int TOK = 64;
  constexpr int TSTR = TOK + 8;  // transposed LDS row stride (u16)
  __shared__ __attribute__((aligned(16))) u16 tr[D * TSTR];
  const int tid = threadIdx.x;
  const int head = blockIdx.y;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * TOK;
  const int64_t rs = static_cast<int64_t>(P.heads) * D;
  // Delta: 4 threads per token, D/4 elements each
  if (P.delta != nullptr) {
    const int t = tid >> 2, part = tid & 3;
    const int64_t row = tok0 + t;
    float acc = 0.f;
    if (row < P.n) {
      const T* op = static_cast<const T*>(P.o) + row * rs + head * D + part * (D / 4);
      const T* gp = static_cast<const T*>(P.d_o) + row * rs + head * D + part * (D / 4);
#pragma unroll
      for (int e = 0; e < D / 4; e += 4) {
        const float4 a = load4(op + e), g = load4(gp + e);
        acc = fmaf(a.x, g.x, acc);
        acc = fmaf(a.y, g.y, acc);
        acc = fmaf(a.z, g.z, acc);
        acc = fmaf(a.w, g.w, acc);
      }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (part == 0 && row < P.n) P.delta[head * P.dpitch + row] = acc;
  }
  if constexpr (sizeof(T) == 2) {
    if (P.qt == nullptr) return;
    const u16* srcs[3] = {static_cast<const u16*>(P.q), static_cast<const u16*>(P.k), static_cast<const u16*>(P.d_o)};
    u16* dsts[3] = {P.qt, P.kt, P.dot};
    constexpr int DCH = D / 8;
#pragma unroll
    for (int which = 0; which < 3; ++which) {
      __syncthreads();
      // [64 tokens][D] -> LDS [D][64]
      for (int ch = tid; ch < TOK * DCH; ch += 256) {
        const int t = ch / DCH, cc = ch % DCH;
        const int64_t row = tok0 + t;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (row < P.n) u = *reinterpret_cast<const uint4*>(srcs[which] + row * rs + head * D + cc * 8);
        const u32 w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tr[(cc * 8 + 2 * e) * TSTR + t] = static_cast<u16>(w[e] & 0xFFFFu);
          tr[(cc * 8 + 2 * e + 1) * TSTR + t] = static_cast<u16>(w[e] >> 16);
        }
      }
      __syncthreads();
      // LDS [D][64] -> rows of 64 tokens (128 bytes) of X^T
      for (int ch = tid; ch < D * (TOK / 8); ch += 256) {
        const int dd = ch / (TOK / 8), c = ch % (TOK / 8);
        const uint4 u = *reinterpret_cast<const uint4*>(tr + dd * TSTR + c * 8);
        *reinterpret_cast<uint4*>(dsts[which] + (static_cast<int64_t>(head) * D + dd) * P.np + tok0 + c * 8) = u;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// bf16 dK/dV.  Workgroup = 8 wave64; each wave owns 32 keys of the item's key block
// (256 keys per workgroup) and keeps their K slices in registers as MFMA B operands
// (V slices in LDS, loaded once: registers hold the dK^T, dV^T accumulators).  The admitted query runs
// are walked in tiles of 32 queries staged in LDS (row-major Q and dO for the score
// products, transposed Q^T and dO^T for the gradient products, plus L and Delta),
// fetched into registers one tile ahead.
//
// Per tile and wave (v_mfma_f32_32x32x16_bf16):
//   S  = Q K^T, dP = dO V^T      A = Q / dO rows read in bit-2/3-swapped order, so the
//                                accumulator value i of a lane (key = lane%32) holds
//                                query 16(i/8) + 8(lane/32) + i%8: exactly the B
//                                operand layout of the next two products
//   P = 2^(S c log2e - L log2e), dS = P (dP - Delta)     (lane-local)
//   dV^T += dO^T P,  dK^T += Q^T dS                      A = 8 consecutive queries of
//                                one dim from the transposed tiles (16-byte reads)
// Query rows past a run's end are staged as zeros with L = +inf, so they give P = 0
// and dS = 0 without masking code.
// ---------------------------------------------------------------------------------
template <int D>
struct BwdKTile {
  static constexpr int NW = 8;
  static constexpr int NT = 64 * NW;
  static constexpr int KB = 32 * NW;      // keys per workgroup
  static constexpr int QT = 32;           // queries per staged tile
  static constexpr int RSTR = D + 8;      // row-major tile stride (u16)
  static constexpr int TSTR = QT + 8;     // transposed tile stride (u16)
  static constexpr int DCH = D / 8;
  static constexpr int ROWB = QT * RSTR * 2;
  static constexpr int TRB = D * TSTR * 2;
  static constexpr int STAGE = 2 * ROWB + 2 * TRB + 2 * QT * 4;
  static constexpr int VBLK = KB * RSTR * 2;  // the workgroup's V rows
  static constexpr int RCH = QT * DCH;    // 16-byte chunks of a row-major tile
  static constexpr int TCH = D * (QT / 8);  // 16-byte chunks of a transposed tile
  static constexpr int RPT = (RCH + NT - 1) / NT;
  static constexpr int TPT = (TCH + NT - 1) / NT;
};

// 8 consecutive tokens [t0, t0 + 8) of one row of a transposed [.][np] array, zero past
// nv (tokens counted from the tile start); 16-byte load when aligned and whole.
__device__ __forceinline__ uint4 load_tr_chunk(const u16* row, int64_t t0, int first, int nv) {
  if (first + 8 <= nv && (t0 & 7) == 0) return *reinterpret_cast<const uint4*>(row + t0);
  u32 w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (first + e < nv) w[e >> 1] |= static_cast<u32>(row[t0 + e]) << (16 * (e & 1));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void attn_bwd_dkdv_bf16(BwdParams P) {
  using T = BwdKTile<D>;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE + T::VBLK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  GroupCoord gc;
  if (!group_coord(blockIdx.x, P.tiles_per_item, P.heads, P.n_items, gc)) return;
  const int tile = gc.tile;
  const int head = gc.head;
  const WorkItem it = P.items[gc.item];
  const KeyRun* runs = P.runs + it.run0;
  const int nrun = it.nrun;
  const int64_t rs = static_cast<int64_t>(P.heads) * D;
  const u16* __restrict__ Q = static_cast<const u16*>(P.q) + head * D;
  const u16* __restrict__ dO = static_cast<const u16*>(P.d_o) + head * D;
  const u16* __restrict__ Qt = P.qt + static_cast<int64_t>(head) * D * P.np;
  const u16* __restrict__ dOt = P.dot + static_cast<int64_t>(head) * D * P.np;
  const float* __restrict__ L = P.lse + head * P.n;
  const float* __restrict__ Dl = P.delta + head * P.n;

  // this lane's key and its K slice (B operand: 8 dims per half-wave per step)
  const int kj = tile * T::KB + wave * 32 + col;
  const bool kok = kj < it.q_len;
  bf16x8 kf[NKK];
  {
    const u16* kp = static_cast<const u16*>(P.k) + (it.q_row0 + (kok ? kj : 0)) * rs + head * D + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 a = make_uint4(0, 0, 0, 0);
      if (kok) a = *reinterpret_cast<const uint4*>(kp + 16 * kk);
      kf[kk] = as_bf16x8(a);
    }
  }
  // the workgroup's V rows -> LDS (read back as B operands of dP = dO V^T)
  u16* vblk = reinterpret_cast<u16*>(smem + 2 * T::STAGE);
  for (int ch = tid; ch < T::KB * T::DCH; ch += T::NT) {
    const int r = ch / T::DCH, cc = ch % T::DCH;
    const int key = tile * T::KB + r;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (key < it.q_len)
      u = *reinterpret_cast<const uint4*>(static_cast<const u16*>(P.v) + (it.q_row0 + key) * rs + head * D + cc * 8);
    *reinterpret_cast<uint4*>(vblk + r * T::RSTR + cc * 8) = u;
  }
  const u16* vrow = vblk + (wave * 32 + col) * T::RSTR + 8 * hl;

  uint4 rq[T::RPT], rg[T::RPT], rqt[T::TPT], rgt[T::TPT];
  float rl = 0.f;
  bool rl_ok = false;
  auto fetch = [&](const TileCursor& c) {
    const int64_t start = c.start + c.k0;
    const int nv = min(T::QT, c.len - c.k0);
#pragma unroll
    for (int i = 0; i < T::RPT; ++i) {
      const int ch = tid + i * T::NT;
      const int r = ch / T::DCH, cc = ch % T::DCH;
      rq[i] = make_uint4(0, 0, 0, 0);
      rg[i] = make_uint4(0, 0, 0, 0);
      if (ch < T::RCH && r < nv) {
        const int64_t off = (start + r) * rs + cc * 8;
        rq[i] = *reinterpret_cast<const uint4*>(Q + off);
        rg[i] = *reinterpret_cast<const uint4*>(dO + off);
      }
    }
#pragma unroll
    for (int i = 0; i < T::TPT; ++i) {
      const int ch = tid + i * T::NT;
      const int dd = ch / (T::QT / 8), c8 = ch % (T::QT / 8);
      rqt[i] = make_uint4(0, 0, 0, 0);
      rgt[i] = make_uint4(0, 0, 0, 0);
      if (ch < T::TCH) {
        rqt[i] = load_tr_chunk(Qt + dd * P.np, start + 8 * c8, 8 * c8, nv);
        rgt[i] = load_tr_chunk(dOt + dd * P.np, start + 8 * c8, 8 * c8, nv);
      }
    }
    // L and Delta of the tile's rows: loaded raw (rows past the run's end read the tile's
    // first row) and turned into their staged values only at the stash, so no
    // instruction here waits for the loads in flight
    if (tid < 2 * T::QT) {
      const int r = tid & (T::QT - 1);
      rl_ok = r < nv;
      rl = (tid < T::QT ? L : Dl)[start + (rl_ok ? r : 0)];
    }
  };
  auto stash = [&](int stage) {
    char* base = smem + stage * T::STAGE;
    u16* qs = reinterpret_cast<u16*>(base);
    u16* gs = reinterpret_cast<u16*>(base + T::ROWB);
    u16* qts = reinterpret_cast<u16*>(base + 2 * T::ROWB);
    u16* gts = reinterpret_cast<u16*>(base + 2 * T::ROWB + T::TRB);
    float* ls = reinterpret_cast<float*>(base + 2 * T::ROWB + 2 * T::TRB);
#pragma unroll
    for (int i = 0; i < T::RPT; ++i) {
      const int ch = tid + i * T::NT;
      const int r = ch / T::DCH, cc = ch % T::DCH;
      if (ch < T::RCH) {
        *reinterpret_cast<uint4*>(qs + r * T::RSTR + cc * 8) = rq[i];
        *reinterpret_cast<uint4*>(gs + r * T::RSTR + cc * 8) = rg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < T::TPT; ++i) {
      const int ch = tid + i * T::NT;
      const int dd = ch / (T::QT / 8), c8 = ch % (T::QT / 8);
      if (ch < T::TCH) {
        *reinterpret_cast<uint4*>(qts + dd * T::TSTR + c8 * 8) = rqt[i];
        *reinterpret_cast<uint4*>(gts + dd * T::TSTR + c8 * 8) = rgt[i];
      }
    }
    if (tid < 2 * T::QT) {
      if (tid < T::QT)
        ls[tid] = rl_ok ? rl * kLog2e : INFINITY;
      else
        ls[tid] = rl_ok ? rl : 0.f;
    }
  };

  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[dt][i] = dv[dt][i] = 0.f;
  const float c2 = P.scale_log2;
  const int prow = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);

  constexpr int kNoCut = 0x3FFFFFFF;  // query runs are never cut (causal masking is below)
  TileCursor cur = cursor_begin(runs, nrun, kNoCut);
  TileCursor nxt = cur;
  int stage = 0;
  if (cur.run < nrun) {
    fetch(cur);
    stash(0);
    cursor_next(nxt, runs, nrun, T::QT, kNoCut);
    if (nxt.run < nrun) fetch(nxt);
  }
  __syncthreads();

  while (cur.run < nrun) {
    const char* base = smem + stage * T::STAGE;
    const u16* qs = reinterpret_cast<const u16*>(base);
    const u16* gs = reinterpret_cast<const u16*>(base + T::ROWB);
    const u16* qts = reinterpret_cast<const u16*>(base + 2 * T::ROWB);
    const u16* gts = reinterpret_cast<const u16*>(base + 2 * T::ROWB + T::TRB);
    const float* ls = reinterpret_cast<const float*>(base + 2 * T::ROWB + 2 * T::TRB);

    f32x16 s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
    {
      const u16* qp = qs + prow * T::RSTR + 8 * hl;
      const u16* gp = gs + prow * T::RSTR + 8 * hl;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * kk)), kf[kk],
                                                     s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(gp + 16 * kk)),
                                                      as_bf16x8(*reinterpret_cast<const uint4*>(vrow + 16 * kk)), dp, 0, 0, 0);
      }
    }
    // causal diagonal run: query k0 + q of the run sees this lane's key kj only if
    // k0 + q >= diag + kj
    if (CAUSAL && cur.diag >= 0 && cur.k0 < cur.diag + (tile + 1) * T::KB) {
      const int lim = cur.diag + kj - cur.k0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * (i >> 3) + 8 * hl + (i & 7) < lim) s[i] = -INFINITY;
    }
    // value i holds query 16*(i/8) + 8*hl + i%8 of the tile (and key col); each half m
    // of the values is turned into P and dS and consumed by
    //   dV^T (dims x keys) += dO^T P ,  dK^T += Q^T dS   (16 queries per step)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float4 l0 = *reinterpret_cast<const float4*>(ls + 16 * m + 8 * hl);
      const float4 l1 = *reinterpret_cast<const float4*>(ls + 16 * m + 8 * hl + 4);
      const float4 d0 = *reinterpret_cast<const float4*>(ls + T::QT + 16 * m + 8 * hl);
      const float4 d1 = *reinterpret_cast<const float4*>(ls + T::QT + 16 * m + 8 * hl + 4);
      const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
      const float dl[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      bf16x8 pb, db;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[8 * m + j], c2, -lv[j]));
        pb[j] = static_cast<__bf16>(p);
        db[j] = static_cast<__bf16>(p * (dp[8 * m + j] - dl[j]));
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int off = (32 * dt + col) * T::TSTR + 16 * m + 8 * hl;
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(gts + off)), pb,
                                                          dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(qts + off)), db,
                                                          dk[dt], 0, 0, 0);
      }
    }

    cur = nxt;
    if (cur.run < nrun) {
      stash(stage ^ 1);
      cursor_next(nxt, runs, nrun, T::QT, kNoCut);
      if (nxt.run < nrun) fetch(nxt);
    }
    stage ^= 1;
    __syncthreads();
  }

  if (kok) {
    const int64_t orow = it.out_row0 + kj;
    float* kp = P.g0 + (orow * P.heads + head) * D;
    float* vp = P.g1 + (orow * P.heads + head) * D;
    const float sc = P.scale;
    // accumulator element i of tile dt holds dim 32*dt + 8*(i/4) + 4*hl + i%4
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * dt + 8 * g + 4 * hl;
        *reinterpret_cast<float4*>(kp + dd) =
            make_float4(sc * dk[dt][4 * g], sc * dk[dt][4 * g + 1], sc * dk[dt][4 * g + 2], sc * dk[dt][4 * g + 3]);
        *reinterpret_cast<float4*>(vp + dd) = make_float4(dv[dt][4 * g], dv[dt][4 * g + 1], dv[dt][4 * g + 2], dv[dt][4 * g + 3]);
      }
  }
}

// ---------------------------------------------------------------------------------
// bf16 dQ.  The forward kernel's shape: 8 wave64 x 32 queries, Q and dO slices in
// registers as B operands, dQ^T accumulated in registers, key tiles of 32 keys staged
// in LDS (row-major K and V for the score products, K^T for the gradient product).
//   S^T = K Q^T, dP^T = V dO^T   (K, V rows in bit-2/3-swapped order: value i of a
//                                 lane (query = lane%32) holds key 16(i/8)+8(lane/32)+i%8)
//   dS^T = P^T (dP^T - Delta)    (L and Delta are per lane)
//   dQ^T += K^T dS^T
// ---------------------------------------------------------------------------------
template <int D>
struct BwdQTile {
  static constexpr int NW = 8;
  static constexpr int NT = 64 * NW;
  static constexpr int QB = 32 * NW;
  static constexpr int KT = 32;
  static constexpr int RSTR = D + 8;
  static constexpr int TSTR = KT + 8;
  static constexpr int DCH = D / 8;
  static constexpr int ROWB = KT * RSTR * 2;
  static constexpr int TRB = D * TSTR * 2;
  static constexpr int STAGE = 2 * ROWB + TRB;
  static constexpr int RCH = KT * DCH;
  static constexpr int TCH = D * (KT / 8);
  static constexpr int RPT = (RCH + NT - 1) / NT;
  static constexpr int TPT = (TCH + NT - 1) / NT;
};

template <int D>
__global__ __launch_bounds__(512) void attn_bwd_dq_bf16(BwdParams P) {
  using T = BwdQTile<D>;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  GroupCoord gc;
  if (!group_coord(blockIdx.x, P.tiles_per_item, P.heads, P.n_items, gc)) return;
  const int tile = gc.tile;
  const int head = gc.head;
  const WorkItem it = P.items[gc.item];
  const KeyRun* runs = P.runs + it.run0;
  const int nrun = it.nrun;
  const int64_t rs = static_cast<int64_t>(P.heads) * D;
  const u16* __restrict__ K = static_cast<const u16*>(P.k) + head * D;
  const u16* __restrict__ V = static_cast<const u16*>(P.v) + head * D;
  const u16* __restrict__ Kt = P.kt + static_cast<int64_t>(head) * D * P.np;

  const int qi = tile * T::QB + wave * 32 + col;
  const bool qok = qi < it.q_len;
  const int64_t qrow = it.q_row0 + (qok ? qi : 0);
  bf16x8 qf[NKK], gf[NKK];
  {
    const int64_t off = qrow * rs + head * D + 8 * hl;
    const u16* qp = static_cast<const u16*>(P.q) + off;
    const u16* gp = static_cast<const u16*>(P.d_o) + off;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 a = make_uint4(0, 0, 0, 0), c = a;
      if (qok) {
        a = *reinterpret_cast<const uint4*>(qp + 16 * kk);
        c = *reinterpret_cast<const uint4*>(gp + 16 * kk);
      }
      qf[kk] = as_bf16x8(a);
      gf[kk] = as_bf16x8(c);
    }
  }
  const float lq = qok ? P.lse[head * P.n + qrow] * kLog2e : INFINITY;
  const float dq_delta = qok ? P.delta[head * P.n + qrow] : 0.f;

  // K/V rows: each thread's chunk sits at a fixed offset from the tile's first row; on a
  // run's ragged last tile rows past the end repeat the run's last row (their scores are
  // masked, so they add nothing).  K^T: 8 consecutive keys of one dim, zero past the run.
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 rk[T::RPT], rv[T::RPT];
  uint4 rkt[T::TPT];
  const uint32_t fcol = (tid % T::DCH) * 8;
  const uint32_t fbase = static_cast<uint32_t>(tid / T::DCH) * static_cast<uint32_t>(rs) + fcol;
  const uint32_t fstep = static_cast<uint32_t>(T::NT / T::DCH) * static_cast<uint32_t>(rs);
  const u16* ktrow[T::TPT];
  int ktc8[T::TPT];
#pragma unroll
  for (int i = 0; i < T::TPT; ++i) {
    const int ch = tid + i * T::NT;
    ktrow[i] = Kt + (ch / (T::KT / 8)) * P.np;
    ktc8[i] = 8 * (ch % (T::KT / 8));
  }
  auto fetch = [&](const TileCursor& c) {
    const int64_t start = c.start + c.k0;
    const int nv = min(T::KT, c.len - c.k0);
    const u16* kb = K + start * rs;
    const u16* vb = V + start * rs;
    const uint32_t last = static_cast<uint32_t>(nv - 1) * static_cast<uint32_t>(rs) + fcol;
#pragma unroll
    for (int i = 0; i < T::RPT; ++i) {
      if (tid + i * T::NT < T::RCH) {
        const uint32_t o = fbase + i * fstep;
        const uint32_t off = o < last ? o : last;
        rk[i] = *reinterpret_cast<const u32x4*>(kb + off);
        rv[i] = *reinterpret_cast<const u32x4*>(vb + off);
      }
    }
#pragma unroll
    for (int i = 0; i < T::TPT; ++i)
      if (tid + i * T::NT < T::TCH) rkt[i] = load_tr_chunk(ktrow[i], start + ktc8[i], ktc8[i], nv);
  };
  auto stash = [&](int stage) {
    char* base = smem + stage * T::STAGE;
    u16* ks = reinterpret_cast<u16*>(base);
    u16* vs = reinterpret_cast<u16*>(base + T::ROWB);
    u16* kts = reinterpret_cast<u16*>(base + 2 * T::ROWB);
#pragma unroll
    for (int i = 0; i < T::RPT; ++i) {
      const int ch = tid + i * T::NT;
      const int r = ch / T::DCH, cc = ch % T::DCH;
      if (ch < T::RCH) {
        *reinterpret_cast<u32x4*>(ks + r * T::RSTR + cc * 8) = rk[i];
        *reinterpret_cast<u32x4*>(vs + r * T::RSTR + cc * 8) = rv[i];
      }
    }
#pragma unroll
    for (int i = 0; i < T::TPT; ++i) {
      const int ch = tid + i * T::NT;
      const int dd = ch / (T::KT / 8), c8 = ch % (T::KT / 8);
      if (ch < T::TCH) *reinterpret_cast<uint4*>(kts + dd * T::TSTR + c8 * 8) = rkt[i];
    }
  };

  f32x16 dq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[dt][i] = 0.f;
  const float c2 = P.scale_log2;
  const int prow = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);

  const int qhi = min(it.q_len, (tile + 1) * T::QB);
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
    const int nv = min(T::KT, cur.len - cur.k0);
    const char* base = smem + stage * T::STAGE;
    const u16* ks = reinterpret_cast<const u16*>(base);
    const u16* vs = reinterpret_cast<const u16*>(base + T::ROWB);
    const u16* kts = reinterpret_cast<const u16*>(base + 2 * T::ROWB);

    // dP^T - Delta: the accumulator starts at -Delta (all 16 values of a lane are its query)
    f32x16 s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = 0.f;
      dp[i] = -dq_delta;
    }
    {
      const u16* kp = ks + prow * T::RSTR + 8 * hl;
      const u16* vp = vs + prow * T::RSTR + 8 * hl;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(kp + 16 * kk)), qf[kk],
                                                     s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(vp + 16 * kk)), gf[kk],
                                                      dp, 0, 0, 0);
      }
    }
    // value i holds key 16*(i/8) + 8*hl + i%8 of the tile; keys past the run are masked
    if (nv < T::KT) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * (i >> 3) + 8 * hl + (i & 7) >= nv) s[i] = -INFINITY;
    }
    // causal diagonal run: this lane's query qi sees key k0 + j only if k0 + j <= diag + qi
    if (cur.diag >= 0 && cur.k0 + T::KT - 1 > cur.diag + tile * T::QB) {
      const int lim = cur.diag + qi - cur.k0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * (i >> 3) + 8 * hl + (i & 7) > lim) s[i] = -INFINITY;
    }
    bf16x8 db[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lq));
      db[i >> 3][i & 7] = static_cast<__bf16>(p * dp[i]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int off = (32 * dt + col) * T::TSTR + 16 * m + 8 * hl;
        dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(kts + off)), db[m],
                                                          dq[dt], 0, 0, 0);
      }
    }

    cur = nxt;
    if (cur.run < nrun) {
      stash(stage ^ 1);
      cursor_next(nxt, runs, nrun, T::KT, qhi);
      if (nxt.run < nrun) fetch(nxt);
    }
    stage ^= 1;
    __syncthreads();
  }

  if (qok) {
    float* gp = P.g0 + ((it.out_row0 + qi) * P.heads + head) * D;
    const float sc = P.scale;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(gp + 32 * dt + 8 * g + 4 * hl) =
            make_float4(sc * dq[dt][4 * g], sc * dq[dt][4 * g + 1], sc * dq[dt][4 * g + 2], sc * dq[dt][4 * g + 3]);
  }
}

// ---------------------------------------------------------------------------------
// float32 backward (correctness path for float32 inputs), fp32 FMA throughout.
// dQ: one wave of 64 queries (one per lane), its Q and dO rows in LDS, 32-key tiles of
// K and V read by broadcast.  dK/dV: 64 keys per workgroup of two waves (wave 0
// accumulates dV, wave 1 dK; both recompute the scores), 32-query tiles of Q, dO, L
// and Delta read by broadcast.
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32(BwdParams P) {
  constexpr int QT = 64, KT = 32, RS = D + 1;
  __shared__ float qs[QT * RS];
  __shared__ float gs[QT * RS];
  __shared__ __attribute__((aligned(16))) float ks[KT * D];
  __shared__ __attribute__((aligned(16))) float vs[KT * D];
  const int lane = threadIdx.x;
  GroupCoord gc;
  if (!group_coord(blockIdx.x, P.tiles_per_item, P.heads, P.n_items, gc)) return;
  const int tile = gc.tile;
  const int head = gc.head;
  const WorkItem it = P.items[gc.item];
  const int64_t rs = static_cast<int64_t>(P.heads) * D;
  const float* Q = static_cast<const float*>(P.q) + head * D;
  const float* G = static_cast<const float*>(P.d_o) + head * D;
  const float* K = static_cast<const float*>(P.k) + head * D;
  const float* V = static_cast<const float*>(P.v) + head * D;
  const int qi = tile * QT + lane;
  const bool qok = qi < it.q_len;
  const int64_t qrow = it.q_row0 + (qok ? qi : 0);
  for (int r = 0; r < QT; ++r) {
    const int qr = tile * QT + r;
    const bool ok = qr < it.q_len;
    for (int t = lane; t < D; t += 64) {
      qs[r * RS + t] = ok ? Q[(it.q_row0 + qr) * rs + t] : 0.f;
      gs[r * RS + t] = ok ? G[(it.q_row0 + qr) * rs + t] : 0.f;
    }
  }
  const float lq = qok ? P.lse[head * P.n + qrow] * kLog2e : INFINITY;
  const float dl = qok ? P.delta[head * P.n + qrow] : 0.f;
  const float c2 = P.scale_log2;
  float dq[D];
#pragma unroll
  for (int t = 0; t < D; ++t) dq[t] = 0.f;
  const int qhi = min(it.q_len, (tile + 1) * QT);
  for (int ri = 0; ri < it.nrun; ++ri) {
    const KeyRun run = P.runs[it.run0 + ri];
    const int rlen = run.diag >= 0 ? min(run.len, run.diag + qhi) : run.len;
    const int lim = run.diag >= 0 ? run.diag + qi : 0x7FFFFFFF;  // causal: keys <= lim
    for (int k0 = 0; k0 < rlen; k0 += KT) {
      const int nv = min(KT, rlen - k0);
      __syncthreads();
      for (int c = lane; c < KT * D; c += 64) {
        const int kr = c / D, kc = c % D;
        ks[c] = kr < nv ? K[(run.start + k0 + kr) * rs + kc] : 0.f;
        vs[c] = kr < nv ? V[(run.start + k0 + kr) * rs + kc] : 0.f;
      }
      __syncthreads();
      for (int j = 0; j < nv; ++j) {
        float s = 0.f, dp = 0.f;
#pragma unroll 8
        for (int t = 0; t < D; ++t) {
          s = fmaf(qs[lane * RS + t], ks[j * D + t], s);
          dp = fmaf(gs[lane * RS + t], vs[j * D + t], dp);
        }
        const float p = k0 + j <= lim ? __builtin_amdgcn_exp2f(fmaf(s, c2, -lq)) : 0.f;
        const float ds = p * (dp - dl);
#pragma unroll
        for (int t = 0; t < D; ++t) dq[t] = fmaf(ds, ks[j * D + t], dq[t]);
      }
    }
  }
  if (qok) {
    float* gp = P.g0 + ((it.out_row0 + qi) * P.heads + head) * D;
#pragma unroll
    for (int t = 0; t < D; ++t) gp[t] = P.scale * dq[t];
  }
}

template <int D>
__global__ __launch_bounds__(128) void attn_bwd_dkdv_f32(BwdParams P) {
  constexpr int KB = 64, QT = 32, RS = D + 1;
  __shared__ float ks[KB * RS];
  __shared__ float vs[KB * RS];
  __shared__ __attribute__((aligned(16))) float qs[QT * D];
  __shared__ __attribute__((aligned(16))) float gs[QT * D];
  __shared__ float ls[QT], dls[QT];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  GroupCoord gc;
  if (!group_coord(blockIdx.x, P.tiles_per_item, P.heads, P.n_items, gc)) return;
  const int tile = gc.tile;
  const int head = gc.head;
  const WorkItem it = P.items[gc.item];
  const int64_t rs = static_cast<int64_t>(P.heads) * D;
  const float* Q = static_cast<const float*>(P.q) + head * D;
  const float* G = static_cast<const float*>(P.d_o) + head * D;
  const float* K = static_cast<const float*>(P.k) + head * D;
  const float* V = static_cast<const float*>(P.v) + head * D;
  const int kj = tile * KB + lane;
  const bool kok = kj < it.q_len;
  for (int c = tid; c < KB * D; c += 128) {
    const int r = c / D, t = c % D;
    const bool ok = tile * KB + r < it.q_len;
    ks[r * RS + t] = ok ? K[(it.q_row0 + tile * KB + r) * rs + t] : 0.f;
    vs[r * RS + t] = ok ? V[(it.q_row0 + tile * KB + r) * rs + t] : 0.f;
  }
  const float c2 = P.scale_log2;
  float acc[D];
#pragma unroll
  for (int t = 0; t < D; ++t) acc[t] = 0.f;
  for (int ri = 0; ri < it.nrun; ++ri) {
    const KeyRun run = P.runs[it.run0 + ri];
    for (int q0 = 0; q0 < run.len; q0 += QT) {
      const int nv = min(QT, run.len - q0);
      __syncthreads();
      for (int c = tid; c < QT * D; c += 128) {
        const int r = c / D, t = c % D;
        qs[c] = r < nv ? Q[(run.start + q0 + r) * rs + t] : 0.f;
        gs[c] = r < nv ? G[(run.start + q0 + r) * rs + t] : 0.f;
      }
      if (tid < QT) {
        ls[tid] = tid < nv ? P.lse[head * P.n + run.start + q0 + tid] * kLog2e : INFINITY;
        dls[tid] = tid < nv ? P.delta[head * P.n + run.start + q0 + tid] : 0.f;
      }
      __syncthreads();
      for (int i = 0; i < nv; ++i) {
        float s = 0.f, dp = 0.f;
#pragma unroll 8
        for (int t = 0; t < D; ++t) {
          s = fmaf(ks[lane * RS + t], qs[i * D + t], s);
          dp = fmaf(vs[lane * RS + t], gs[i * D + t], dp);
        }
        // causal diagonal run: query q0 + i sees this lane's key kj only if q0 + i >= diag + kj
        const bool vis = run.diag < 0 || q0 + i >= run.diag + kj;
        const float p = vis ? __builtin_amdgcn_exp2f(fmaf(s, c2, -ls[i])) : 0.f;
        if (wave == 0) {
#pragma unroll
          for (int t = 0; t < D; ++t) acc[t] = fmaf(p, gs[i * D + t], acc[t]);
        } else {
          const float ds = p * (dp - dls[i]);
#pragma unroll
          for (int t = 0; t < D; ++t) acc[t] = fmaf(ds, qs[i * D + t], acc[t]);
        }
      }
    }
  }
  if (kok) {
    const int64_t orow = it.out_row0 + kj;
    float* gp = (wave == 0 ? P.g1 : P.g0) + (orow * P.heads + head) * D;
    const float sc = wave == 0 ? 1.f : P.scale;
#pragma unroll
    for (int t = 0; t < D; ++t) gp[t] = sc * acc[t];
  }
}

// ---------------------------------------------------------------------------------
// Sum of the visit slots of a gradient in slot order, rounded to the output dtype.
// ---------------------------------------------------------------------------------
template <typename OutT>
__global__ __launch_bounds__(256) void sum_slots(const float* __restrict__ in, int64_t stride, int nslot,
                                                 int64_t count4, OutT* __restrict__ out) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < count4;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    float4 a = *reinterpret_cast<const float4*>(in + 4 * e);
    for (int s = 1; s < nslot; ++s) {
      const float4 c = *reinterpret_cast<const float4*>(in + s * stride + 4 * e);
      a.x += c.x;
      a.y += c.y;
      a.z += c.z;
      a.w += c.w;
    }
    store_out(out + 4 * e, a);
  }
}

// ---------------------------------------------------------------------------------
// Accumulation of one visit's gradient terms (stream engine): a = term on a row's first
// visit, else a = acc + term -- the order of the device path's slot sum; the result goes
// back to acc, or, at the last visit, to out in the output dtype.
// ---------------------------------------------------------------------------------
template <typename OutT>
__global__ __launch_bounds__(256) void accumulate_terms(float* __restrict__ acc, const float* __restrict__ term,
                                                        int64_t count4, int first, OutT* __restrict__ out) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < count4;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    float4 a = *reinterpret_cast<const float4*>(term + 4 * e);
    if (!first) {
      const float4 c = *reinterpret_cast<const float4*>(acc + 4 * e);
      a = make_float4(c.x + a.x, c.y + a.y, c.z + a.z, c.w + a.w);
    }
    if (out != nullptr)
      store_out(out + 4 * e, a);
    else
      *reinterpret_cast<float4*>(acc + 4 * e) = a;
  }
}

}  // namespace

hipError_t launch_accumulate(const AccLaunch& a, hipStream_t stream) {
  if (a.count <= 0) return hipSuccess;
  if (a.count % 4 != 0) return hipErrorInvalidValue;
  const int64_t count4 = a.count / 4;
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>((count4 + 255) / 256, 65536)));
  if (a.out == nullptr)
    hipLaunchKernelGGL((accumulate_terms<float>), grid, dim3(256), 0, stream, a.acc, a.term, count4, a.first ? 1 : 0,
                       static_cast<float*>(nullptr));
  else if (a.dtype == CQSA_BF16)
    hipLaunchKernelGGL((accumulate_terms<u16>), grid, dim3(256), 0, stream, a.acc, a.term, count4, a.first ? 1 : 0,
                       static_cast<u16*>(a.out));
  else
    hipLaunchKernelGGL((accumulate_terms<float>), grid, dim3(256), 0, stream, a.acc, a.term, count4, a.first ? 1 : 0,
                       static_cast<float*>(a.out));
  return hipGetLastError();
}

int bwd_key_tile(cqsa_dtype dtype) { return dtype == CQSA_BF16 ? BwdKTile<128>::KB : 64; }
int bwd_query_tile(cqsa_dtype dtype) { return dtype == CQSA_BF16 ? BwdQTile<128>::QB : 64; }

hipError_t launch_bwd_prep(const PrepLaunch& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  PrepParams p;
  p.q = a.q;
  p.k = a.k;
  p.o = a.o;
  p.d_o = a.d_o;
  p.delta = a.delta;
  p.qt = static_cast<u16*>(a.qt);
  p.kt = static_cast<u16*>(a.kt);
  p.dot = static_cast<u16*>(a.dot);
  p.n = a.n;
  p.np = a.np;
  p.dpitch = a.dpitch > 0 ? a.dpitch : a.n;
  p.heads = a.heads;
  const int64_t tiles = (a.n + 63) / 64;
  if (tiles > 0x7FFFFFFF || a.heads > 65535) return hipErrorInvalidConfiguration;
  if (a.dtype == CQSA_BF16 && a.qt != nullptr && (a.np < tiles * 64 || (a.np & 7) != 0)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.heads));
  if (a.dtype == CQSA_BF16) {
    if (a.d == 128)
      hipLaunchKernelGGL((bwd_prep<128, u16>), grid, dim3(256), 0, stream, p);
    else if (a.d == 64)
      hipLaunchKernelGGL((bwd_prep<64, u16>), grid, dim3(256), 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL((bwd_prep<128, float>), grid, dim3(256), 0, stream, p);
    else if (a.d == 64)
      hipLaunchKernelGGL((bwd_prep<64, float>), grid, dim3(256), 0, stream, p);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

namespace {

BwdParams bwd_params(const BwdLaunch& a) {
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.d_o = a.d_o;
  p.qt = static_cast<const u16*>(a.qt);
  p.kt = static_cast<const u16*>(a.kt);
  p.dot = static_cast<const u16*>(a.dot);
  p.lse = a.lse;
  p.delta = a.delta;
  p.items = a.items;
  p.runs = a.runs;
  p.n = a.n;
  p.np = a.np;
  p.heads = a.heads;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  p.g0 = nullptr;
  p.g1 = nullptr;
  p.n_items = 0;
  p.tiles_per_item = 0;
  return p;
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdLaunch& a, hipStream_t stream) {
  if (a.n_kitems <= 0 || a.q_len <= 0) return hipSuccess;
  BwdParams p = bwd_params(a);
  p.g0 = a.dk_out;
  p.g1 = a.dv_out;
  p.items = a.kitems;
  p.runs = a.kruns;
  p.n_items = a.n_kitems;
  const int kb = bwd_key_tile(a.dtype);
  p.tiles_per_item = (a.q_len + kb - 1) / kb;
  const int64_t blocks = group_grid(int64_t(a.n_kitems) * a.heads, p.tiles_per_item);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a.dtype == CQSA_BF16) {
    if (a.d == 128 && a.causal)
      hipLaunchKernelGGL((attn_bwd_dkdv_bf16<128, true>), grid, dim3(BwdKTile<128>::NT), 0, stream, p);
    else if (a.d == 128)
      hipLaunchKernelGGL((attn_bwd_dkdv_bf16<128, false>), grid, dim3(BwdKTile<128>::NT), 0, stream, p);
    else if (a.d == 64 && a.causal)
      hipLaunchKernelGGL((attn_bwd_dkdv_bf16<64, true>), grid, dim3(BwdKTile<64>::NT), 0, stream, p);
    else if (a.d == 64)
      hipLaunchKernelGGL((attn_bwd_dkdv_bf16<64, false>), grid, dim3(BwdKTile<64>::NT), 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL(attn_bwd_dkdv_f32<128>, grid, dim3(128), 0, stream, p);
    else if (a.d == 64)
      hipLaunchKernelGGL(attn_bwd_dkdv_f32<64>, grid, dim3(128), 0, stream, p);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdLaunch& a, hipStream_t stream) {
  if (a.n_items <= 0 || a.q_len <= 0) return hipSuccess;
  BwdParams p = bwd_params(a);
  p.g0 = a.dq_out;
  p.n_items = a.n_items;
  const int qb = bwd_query_tile(a.dtype);
  p.tiles_per_item = (a.q_len + qb - 1) / qb;
  const int64_t blocks = group_grid(int64_t(a.n_items) * a.heads, p.tiles_per_item);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a.dtype == CQSA_BF16) {
    if (a.d == 128)
      hipLaunchKernelGGL(attn_bwd_dq_bf16<128>, grid, dim3(BwdQTile<128>::NT), 0, stream, p);
    else if (a.d == 64)
      hipLaunchKernelGGL(attn_bwd_dq_bf16<64>, grid, dim3(BwdQTile<64>::NT), 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL(attn_bwd_dq_f32<128>, grid, dim3(64), 0, stream, p);
    else if (a.d == 64)
      hipLaunchKernelGGL(attn_bwd_dq_f32<64>, grid, dim3(64), 0, stream, p);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sum_slots(const SumLaunch& a, hipStream_t stream) {
  const int64_t count = a.rows * a.heads * a.d;
  if (count <= 0) return hipSuccess;
  if (count % 4 != 0 || a.nslot < 1) return hipErrorInvalidValue;
  const int64_t count4 = count / 4;
  const int64_t blocks = std::min<int64_t>((count4 + 255) / 256, 65536);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a.dtype == CQSA_BF16)
    hipLaunchKernelGGL((sum_slots<u16>), grid, dim3(256), 0, stream, a.in, a.stride, a.nslot, count4,
                       static_cast<u16*>(a.out));
  else
    hipLaunchKernelGGL((sum_slots<float>), grid, dim3(256), 0, stream, a.in, a.stride, a.nslot, count4,
                       static_cast<float*>(a.out));
  return hipGetLastError();
}

}  // namespace cqsa
