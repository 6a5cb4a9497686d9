// Host CQS planner.
//
// Combinatorics follow "Stream-CQSA: Breaking the Billion-Token Barrier on a Single
// GPU" (wispaper explainer): section "The 'CQS Divide': Attention as a Steiner System"
// (c = l(l-1)+1 chunks, c subsequences of l chunks, every chunk pair exactly once),
// section "The Recursive Benefit" (divide a task again), and section "Implementation:
// From High-Level Logic to GPU Kernels" (a CQS Mask removes the redundant overlapping
// regions).  The construction rule of the quorum (cyclic quorum sets, per the abstract of
// arXiv 2604.20819) and the owner of each diagonal block are
// readings: the smallest perfect difference set containing {0,1}, and "chunk x owns its
// diagonal block in task t = x".
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <thread>

namespace cqsa {

namespace {

bool dfs_extend(int l, int c, std::vector<int>& chosen, std::vector<char>& used, int start) {
  if (static_cast<int>(chosen.size()) == l) return true;
  for (int x = start; x < c; ++x) {
    // both differences against every chosen residue must be unused so far
    std::vector<int> fresh;
    bool ok = true;
    for (int a : chosen) {
      const int d1 = (x - a + c) % c, d2 = (a - x + c) % c;
      if (used[d1] || used[d2] || d1 == d2 ||
          std::find(fresh.begin(), fresh.end(), d1) != fresh.end() ||
          std::find(fresh.begin(), fresh.end(), d2) != fresh.end()) {
        ok = false;
        break;
      }
      fresh.push_back(d1);
      fresh.push_back(d2);
    }
    if (!ok) continue;
    chosen.push_back(x);
    for (int f : fresh) used[f] = 1;
    if (dfs_extend(l, c, chosen, used, x + 1)) return true;
    for (int f : fresh) used[f] = 0;
    chosen.pop_back();
  }
  return false;
}

}  // namespace

cqsa_status difference_set(int l, std::vector<int>& out, std::string& why) {
  out.clear();
  if (l < 1 || l > CQSA_MAX_L) {
    why = "l must be in 1.." + std::to_string(CQSA_MAX_L);
    return CQSA_EINVAL;
  }
  if (l == 1) {
    out.push_back(0);
    return CQSA_OK;
  }
  const int c = l * (l - 1) + 1;
  // The search is deterministic and takes tens of milliseconds for l = 10, so each l is
  // searched once per process and its result kept.
  static std::mutex mu;
  static std::vector<int> found[CQSA_MAX_L + 1];
  static int state[CQSA_MAX_L + 1] = {};  // 0 not searched, 1 found, -1 none exists
  std::lock_guard<std::mutex> lock(mu);
  if (state[l] == 0) {
    std::vector<char> used(c, 0);
    std::vector<int> chosen{0, 1};
    used[1] = used[c - 1] = 1;
    state[l] = dfs_extend(l, c, chosen, used, 2) ? 1 : -1;
    if (state[l] == 1) found[l] = chosen;
  }
  if (state[l] < 0) {
    why = "no perfect difference set exists for l=" + std::to_string(l) + " (c=" + std::to_string(c) + ")";
    return CQSA_ENOSET;
  }
  out = found[l];
  return CQSA_OK;
}

StreamLayout stream_layout(const Plan& p, bool acc_on_device, int kv_buffers) {
  StreamLayout s{};
  const int64_t u = p.unit, h = p.heads, d = p.d, e = p.elem_bytes();
  s.kv_stage = align_up(p.task_tokens() * p.row_in_bytes());
  s.q_blk = align_up(u * p.row_in_bytes());
  s.n_blk = align_up(u * h * d * 4);
  s.ml_blk = align_up(u * h * 2 * 4);
  s.o_blk = align_up(u * h * d * e);
  // LSE of every row stays on the device (one copy back at the end) while it is a small
  // share of the budget; otherwise each finished block's LSE goes back per head
  const int64_t lse_all = align_up(h * p.n * 4);
  const bool resident = p.budget == 0 || lse_all <= p.budget / 16;
  s.lse_all = resident ? lse_all : 0;
  s.lse_blk = resident ? 0 : align_up(h * u * 4);
  s.acc_n = acc_on_device ? align_up(p.n * h * d * 4) : 0;
  s.acc_ml = acc_on_device ? align_up(p.n * h * 2 * 4) : 0;
  const int64_t slot = s.q_blk + s.n_blk + s.ml_blk + (acc_on_device ? 0 : s.n_blk + s.ml_blk) + s.o_blk + s.lse_blk;
  s.total = 2 * kv_buffers * s.kv_stage + 2 * slot + s.lse_all + s.acc_n + s.acc_ml;
  return s;
}

BwdLayout bwd_layout(const Plan& p) {
  BwdLayout b{};
  b.delta = align_up(int64_t(p.heads) * p.n * 4);
  b.trans = p.dtype == CQSA_BF16 ? align_up(int64_t(p.heads) * p.d * p.bwd_np * 2) : 0;
  b.slots = align_up(p.visits * p.n * p.heads * int64_t(p.d) * 4);
  b.total = b.delta + 3 * b.trans + 3 * b.slots;
  return b;
}

BwdStreamLayout bwd_stream_layout(const Plan& p, bool acc_on_device, int stage_sets, bool host_stats) {
  BwdStreamLayout b{};
  b.sets = stage_sets;
  b.host_stats = host_stats;
  const int64_t h = p.heads, d = p.d, e = p.elem_bytes(), T = p.task_tokens(), U = p.unit;
  b.tnp = (T + 63) / 64 * 64;
  b.lse = host_stats ? 0 : align_up(h * p.n * 4);
  b.delta = b.lse;
  b.stage = align_up(T * h * d * e);
  b.trans = p.dtype == CQSA_BF16 ? align_up(h * d * b.tnp * 2) : 0;
  b.tstat = align_up(h * T * 4);
  b.term = align_up(U * h * d * 4);
  b.temp = acc_on_device ? 0 : b.term;
  b.out = align_up(U * h * d * e);
  b.acc = acc_on_device ? align_up(p.n * h * d * 4) : 0;
  b.total = b.lse + b.delta + stage_sets * (4 * b.stage + 3 * b.trans + 2 * b.tstat) + 2 * 3 * (b.term + b.temp + b.out) +
            3 * b.acc;
  return b;
}

namespace {

constexpr uint32_t kKnownFlags =
    CQSA_FLAG_HOST_ACC | CQSA_FLAG_KV_SINGLE | CQSA_FLAG_PAD | CQSA_FLAG_CAUSAL | CQSA_FLAG_FREE_BUDGET;

// Every innermost task with its units, per-level chunk of each local unit, admitted
// runs and segments.  With several levels a (task, query unit) may admit no key at all
// (its keys all belong to other tasks); its partial is then the empty triple.
cqsa_status build_tasks(Plan& p, std::string& why) {
  (void)why;
  const bool causal = (p.flags & CQSA_FLAG_CAUSAL) != 0;
  const int levels = static_cast<int>(p.ls.size());
  std::vector<int64_t> parent_len(levels + 1), chunk_len(levels);
  parent_len[0] = p.n_units;
  for (int k = 0; k < levels; ++k) {
    chunk_len[k] = parent_len[k] / p.cs[k];
    parent_len[k + 1] = chunk_len[k] * p.ls[k];
  }
  p.task_units = parent_len[levels];
  // sorted member chunks of every subsequence, per level
  std::vector<std::vector<std::vector<int>>> members(levels);
  for (int k = 0; k < levels; ++k) {
    members[k].resize(p.cs[k]);
    for (int t = 0; t < p.cs[k]; ++t) {
      for (int dd : p.sets[k]) members[k][t].push_back((t + dd) % p.cs[k]);
      std::sort(members[k][t].begin(), members[k][t].end());
    }
  }
  const int64_t n_tasks = p.n_units;  // prod(c)
  p.tasks.assign(n_tasks, Task{});
  const int64_t tu = p.task_units;
  // Every task is built independently (its units, the CQS Mask over its unit pairs, its
  // segments); large plans spread the tasks over host threads.  Only the visit slots
  // depend on the task order, so they are numbered afterwards in ascending task id.
  auto build_range = [&](int64_t t0, int64_t t1) {
    std::vector<int32_t> chunk_of(static_cast<size_t>(levels) * tu);
    for (int64_t tid = t0; tid < t1; ++tid) {
      Task& task = p.tasks[tid];
      task.tid = tid;
      task.ids.assign(levels, 0);
      int64_t rem = tid;
      for (int k = levels - 1; k >= 0; --k) {
        task.ids[k] = static_cast<int>(rem % p.cs[k]);
        rem /= p.cs[k];
      }
      task.units.resize(tu);
      for (int64_t a = 0; a < tu; ++a) {
        int64_t x = a;  // index in the level-k task list, walking outward
        for (int k = levels - 1; k >= 0; --k) {
          const int chunk = members[k][task.ids[k]][x / chunk_len[k]];
          chunk_of[static_cast<size_t>(k) * tu + a] = chunk;
          x = chunk * chunk_len[k] + x % chunk_len[k];
        }
        task.units[a] = x;
      }
      // CQS Mask: admitted iff at every level the chunks differ or equal the task's own index
      task.runs.assign(tu, {});
      for (int64_t a = 0; a < tu; ++a) {
        auto& runs = task.runs[a];
        for (int64_t b = 0; b < tu; ++b) {
          bool ok = true;
          for (int k = 0; k < levels && ok; ++k) {
            const int ca = chunk_of[static_cast<size_t>(k) * tu + a];
            const int cb = chunk_of[static_cast<size_t>(k) * tu + b];
            ok = (ca != cb) || (ca == task.ids[k]);
          }
          if (!ok || (causal && b > a)) continue;
          ++task.admitted_units;
          if (!runs.empty() && runs.back().start + runs.back().count == b)
            ++runs.back().count;
          else
            runs.push_back({static_cast<int32_t>(b), 1});
        }
      }
      for (int64_t a = 0; a < tu; ++a) {
        const int64_t g = task.units[a];
        if (!task.segments.empty() &&
            task.segments.back().global_start + task.segments.back().length == g * p.unit)
          task.segments.back().length += p.unit;
        else
          task.segments.push_back({g * p.unit, p.unit, a * p.unit});
      }
      // padding (CQSA_FLAG_PAD): cut every segment at N, drop those that start past it
      std::vector<Segment> real;
      for (const Segment& g : task.segments)
        if (g.global_start < p.n) real.push_back({g.global_start, std::min(g.length, p.n - g.global_start), g.local_offset});
      task.segments.swap(real);
    }
  };
  const int64_t cells = n_tasks * tu * tu * levels;
  const int64_t workers = cells < (int64_t(1) << 24)
                              ? 1
                              : std::max<int64_t>(1, std::min<int64_t>({16, int64_t(std::thread::hardware_concurrency()),
                                                                        n_tasks}));
  if (workers == 1) {
    build_range(0, n_tasks);
  } else {
    std::vector<std::thread> pool;
    const int64_t per = (n_tasks + workers - 1) / workers;
    for (int64_t w = 0; w < workers; ++w) {
      const int64_t t0 = w * per, t1 = std::min(n_tasks, t0 + per);
      if (t0 < t1) pool.emplace_back(build_range, t0, t1);
    }
    for (auto& th : pool) th.join();
  }
  std::vector<int32_t> seen(p.n_units, 0);
  for (Task& task : p.tasks) {
    task.slot.resize(tu);
    for (int64_t a = 0; a < tu; ++a) task.slot[a] = seen[task.units[a]]++;
  }
  return CQSA_OK;
}

void build_schedule(Plan& p) {
  auto& s = p.schedule;
  s.clear();
  s.push_back(static_cast<int64_t>(p.ls.size()));
  for (size_t k = 0; k < p.ls.size(); ++k) {
    s.push_back(p.cs[k]);
    s.push_back(p.ls[k]);
  }
  s.push_back(static_cast<int64_t>(p.tasks.size()));
  s.push_back(p.unit);
  s.push_back(p.n_units);
  for (const Task& t : p.tasks) {
    s.push_back(t.tid);
    for (int id : t.ids) s.push_back(id);
    s.push_back(static_cast<int64_t>(t.segments.size()));
    for (const Segment& g : t.segments) {
      s.push_back(g.global_start);
      s.push_back(g.length);
      s.push_back(g.local_offset);
    }
    s.push_back(static_cast<int64_t>(t.units.size()));
    for (size_t a = 0; a < t.units.size(); ++a) {
      s.push_back(t.units[a]);
      s.push_back(static_cast<int64_t>(t.runs[a].size()));
      for (const UnitRun& r : t.runs[a]) {
        s.push_back(r.start);
        s.push_back(r.count);
      }
    }
  }
}

// Does task t admit local units (a, b) (in either role; the CQS Mask is symmetric)?
bool admitted_pair(const Plan& p, const Task& t, int64_t a, int64_t b) {
  for (const UnitRun& r : t.runs[a])
    if (b >= r.start && b < r.start + r.count) return true;
  // causal runs of a stop at a: look at b's runs for a (b > a)
  for (const UnitRun& r : t.runs[b])
    if (a >= r.start && a < r.start + r.count) return true;
  (void)p;
  return false;
}

// Dispatch order of a causal plan's device-resident partial launch.  Its workgroups
// differ in work (a query tile sees its diagonal run only up to its own rows, so the
// later tiles of an item see more keys), and the hardware deals workgroup b to XCD b % 8;
// with whole chunks dealt round-robin, the chunk count and their uneven work leave some
// XCDs idle at the end.  Here the chunks (the kernel's cut of each (item, head) group into
// chunks of at most kDispatchChunk tiles, which keeps a chunk's K/V stream in one L2) go
// heaviest first to the XCD with the least work, and inside a chunk the heavier tiles go
// first.  Entry 8k + x is the k-th workgroup of XCD x.  Work of a tile: its 64-key (bf16)
// or 32-key tiles after the causal cut, plus four for the workgroup's fixed cost.  The
// order changes no result, only which workgroup runs where and when.
void build_dispatch(Plan& p) {
  p.dev_order.clear();
  const bool bf = p.dtype == CQSA_BF16;
  const int64_t qt = bf ? kAttnQueryTileBf16 : kAttnQueryTileF32, kt = bf ? kAttnKeyTileBf16 : kAttnKeyTileF32;
  const int64_t tiles = (p.unit + qt - 1) / qt, items = static_cast<int64_t>(p.dev_items.size());
  const int64_t wgs = items * p.heads * tiles;
  if (wgs == 0 || wgs + 8 * kDispatchChunk > kMaxDispatchEntries) return;  // arithmetic order
  const int64_t per = (tiles + kDispatchChunk - 1) / kDispatchChunk, ct = (tiles + per - 1) / per;
  std::vector<int64_t> work(items * tiles);
  for (int64_t i = 0; i < items; ++i) {
    const WorkItem& it = p.dev_items[i];
    for (int64_t t = 0; t < tiles; ++t) {
      const int64_t qhi = std::min<int64_t>(it.q_len, (t + 1) * qt);
      int64_t w = 4;
      for (int32_t r = it.run0; r < it.run0 + it.nrun; ++r) {
        const KeyRun& run = p.dev_runs[r];
        const int64_t len = run.diag >= 0 ? std::min<int64_t>(run.len, run.diag + qhi) : run.len;
        if (len > 0) w += (len + kt - 1) / kt;
      }
      work[i * tiles + t] = w;
    }
  }
  struct Chunk {
    int64_t work, group, first, count;
  };
  std::vector<Chunk> chunks;
  for (int64_t g = 0; g < items * p.heads; ++g)
    for (int64_t c = 0; c < per; ++c) {
      const int64_t first = c * ct, count = std::min(tiles, first + ct) - first;
      if (count <= 0) continue;
      int64_t w = 0;
      for (int64_t t = first; t < first + count; ++t) w += work[(g / p.heads) * tiles + t];
      chunks.push_back({w, g, first, count});
    }
  std::stable_sort(chunks.begin(), chunks.end(), [](const Chunk& a, const Chunk& b) { return a.work > b.work; });
  std::vector<std::vector<int32_t>> seq(8);
  int64_t load[8] = {};
  std::vector<int64_t> order;
  for (const Chunk& ch : chunks) {
    const int x = static_cast<int>(std::min_element(load, load + 8) - load);
    load[x] += ch.work;
    order.clear();
    for (int64_t t = ch.first; t < ch.first + ch.count; ++t) order.push_back(t);
    const int64_t item = ch.group / p.heads;
    std::stable_sort(order.begin(), order.end(),
                     [&](int64_t a, int64_t b) { return work[item * tiles + a] > work[item * tiles + b]; });
    for (int64_t t : order) seq[x].push_back(static_cast<int32_t>(ch.group * tiles + t));
  }
  size_t rounds = 0;
  for (const auto& q : seq) rounds = std::max(rounds, q.size());
  p.dev_order.assign(8 * rounds, -1);
  for (int x = 0; x < 8; ++x)
    for (size_t k = 0; k < seq[x].size(); ++k) p.dev_order[8 * k + x] = seq[x][k];
}

// Kernel descriptor tables.  Key runs are split wherever the task's local order is not
// globally contiguous, in both tables, so device-resident and streamed execution walk
// identical key tiles and give identical bits.
void build_descriptors(Plan& p) {
  const bool causal = (p.flags & CQSA_FLAG_CAUSAL) != 0;
  p.bstream_items.clear();
  p.dev_items.clear();
  p.dev_runs.clear();
  p.stream_items.clear();
  p.stream_runs.clear();
  for (const Task& t : p.tasks) {
    for (size_t a = 0; a < t.units.size(); ++a) {
      WorkItem di{}, si{};
      di.q_row0 = t.units[a] * p.unit;
      di.out_row0 = int64_t(t.slot[a]) * p.n + t.units[a] * p.unit;
      di.q_len = si.q_len = static_cast<int32_t>(p.unit_rows(t.units[a]));
      di.run0 = static_cast<int32_t>(p.dev_runs.size());
      si.run0 = static_cast<int32_t>(p.stream_runs.size());
      int64_t keys = 0;
      for (const UnitRun& r : t.runs[a]) {
        int64_t b = r.start;
        const int64_t end = r.start + r.count;
        while (b < end) {
          int64_t e = b + 1;
          while (e < end && t.units[e] == t.units[e - 1] + 1) ++e;
          // keys at or past N are padding: clip the run there (units are ascending in it)
          const int64_t len = std::min((e - b) * p.unit, p.n - t.units[b] * p.unit);
          // causal: the piece that ends with the query unit itself holds the diagonal
          const int32_t diag = causal && e == static_cast<int64_t>(a) + 1 ? static_cast<int32_t>((static_cast<int64_t>(a) - b) * p.unit) : -1;
          if (len > 0) {
            p.dev_runs.push_back({t.units[b] * p.unit, static_cast<int32_t>(len), diag});
            p.stream_runs.push_back({b * p.unit, static_cast<int32_t>(len), diag});
            keys += len;
          }
          b = e;
        }
      }
      di.nrun = si.nrun = static_cast<int32_t>(p.dev_runs.size()) - di.run0;
      di.keys = si.keys = static_cast<int32_t>(std::min<int64_t>(keys, INT32_MAX));
      if (di.q_len > 0) p.dev_items.push_back(di);  // a unit of padding only has no rows
      p.stream_items.push_back(si);                 // indexed by (task, unit): kept, engine skips it
      WorkItem bi = si;
      bi.q_row0 = static_cast<int64_t>(a) * p.unit;
      p.bstream_items.push_back(bi);
    }
  }
  // heaviest query blocks first in the one-launch device path (load balance only)
  std::stable_sort(p.dev_items.begin(), p.dev_items.end(),
                   [](const WorkItem& x, const WorkItem& y) { return x.keys > y.keys; });
  p.dev_order.clear();
  if (causal) build_dispatch(p);

  p.dev_kitems.clear();
  p.dev_kruns.clear();
  p.bstream_kitems.clear();
  p.bstream_kruns.clear();
  if (!causal) return;
  for (const Task& t : p.tasks) {
    const int64_t tu = static_cast<int64_t>(t.units.size());
    for (int64_t a = 0; a < tu; ++a) {
      WorkItem ki{};
      ki.q_row0 = t.units[a] * p.unit;
      ki.out_row0 = int64_t(t.slot[a]) * p.n + t.units[a] * p.unit;
      ki.q_len = static_cast<int32_t>(p.unit_rows(t.units[a]));
      ki.run0 = static_cast<int32_t>(p.dev_kruns.size());
      WorkItem ks{};
      ks.q_row0 = a * p.unit;
      ks.q_len = ki.q_len;
      ks.run0 = static_cast<int32_t>(p.bstream_kruns.size());
      int64_t rows = 0;
      // query units b >= a that the task admits with a (the mask is symmetric in a, b)
      int64_t b = a;
      while (b < tu) {
        if (!admitted_pair(p, t, a, b)) {
          ++b;
          continue;
        }
        int64_t e = b + 1;
        while (e < tu && t.units[e] == t.units[e - 1] + 1 && admitted_pair(p, t, a, e)) ++e;
        const int64_t len = std::min((e - b) * p.unit, p.n - t.units[b] * p.unit);
        if (len > 0) {
          p.dev_kruns.push_back({t.units[b] * p.unit, static_cast<int32_t>(len), b == a ? 0 : -1});
          p.bstream_kruns.push_back({b * p.unit, static_cast<int32_t>(len), b == a ? 0 : -1});
          rows += len;
        }
        b = e;
      }
      ki.nrun = static_cast<int32_t>(p.dev_kruns.size()) - ki.run0;
      ki.keys = static_cast<int32_t>(std::min<int64_t>(rows, INT32_MAX));
      ks.nrun = ki.nrun;
      ks.keys = ki.keys;
      if (ki.q_len > 0) p.dev_kitems.push_back(ki);
      p.bstream_kitems.push_back(ks);  // indexed by (task, unit)
    }
  }
  std::stable_sort(p.dev_kitems.begin(), p.dev_kitems.end(),
                   [](const WorkItem& x, const WorkItem& y) { return x.keys > y.keys; });
}

}  // namespace

int64_t descriptor_bytes(const Plan& p) {
  return align_up(int64_t(p.dev_order.size()) * int64_t(sizeof(int32_t))) +
         align_up(int64_t(p.dev_items.size()) * sizeof(WorkItem)) +
         align_up(int64_t(p.dev_runs.size()) * sizeof(KeyRun)) +
         align_up(int64_t(p.dev_kitems.size()) * sizeof(WorkItem)) +
         align_up(int64_t(p.dev_kruns.size()) * sizeof(KeyRun)) +
         align_up(int64_t(p.bstream_items.size()) * sizeof(WorkItem)) +
         align_up(int64_t(p.bstream_kitems.size()) * sizeof(WorkItem)) +
         align_up(int64_t(p.bstream_kruns.size()) * sizeof(KeyRun)) +
         align_up(int64_t(p.stream_items.size()) * sizeof(WorkItem)) +
         align_up(int64_t(p.stream_runs.size()) * sizeof(KeyRun));
}

namespace {

// The one budget test of every staging layout (forward and backward, plan and dry run):
// the layout's workspace plus the plan's descriptor tables fit the budget.
bool fits_budget(const Plan& p, int64_t workspace_bytes) {
  return p.budget == 0 || workspace_bytes + descriptor_bytes(p) <= p.budget;
}

cqsa_status choose_mode(Plan& p, std::string& why) {
  struct Cand {
    bool dev;
    int kv;
  };
  const Cand order[4] = {{true, 2}, {false, 2}, {true, 1}, {false, 1}};
  int64_t smallest = -1;
  for (const Cand& c : order) {
    if ((p.flags & CQSA_FLAG_HOST_ACC) && c.dev) continue;
    if ((p.flags & CQSA_FLAG_KV_SINGLE) && c.kv != 1) continue;
    const int64_t bytes = stream_layout(p, c.dev, c.kv).total;
    if (smallest < 0 || bytes < smallest) smallest = bytes;
    if (fits_budget(p, bytes)) {
      p.stream_fp = {c.dev, c.kv, bytes};
      p.host_acc_bytes = c.dev ? 0 : p.n * p.row_part_bytes();
      return CQSA_OK;
    }
  }
  why = "no staging mode fits the budget of " + std::to_string(p.budget) + " bytes (smallest needs " +
        std::to_string(smallest + descriptor_bytes(p)) + ")";
  return CQSA_EBUDGET;
}

// Levels, difference sets, unit grid and visit count of a plan; no task is built.
cqsa_status plan_shape(int64_t n, int heads, int d, cqsa_dtype dtype, const std::vector<int>& ls, int64_t budget,
                       uint32_t flags, Plan& p, std::string& why) {
  p.n = n;
  p.heads = heads;
  p.d = d;
  p.dtype = dtype;
  p.ls = ls;
  p.cs.clear();
  p.sets.clear();
  p.budget = budget;
  p.flags = flags;
  int64_t prod_c = 1, prod_l = 1;
  for (int l : ls) {
    std::vector<int> dset;
    const cqsa_status st = difference_set(l, dset, why);
    if (st != CQSA_OK) return st;
    p.sets.push_back(dset);
    p.cs.push_back(l * (l - 1) + 1);
    prod_c *= p.cs.back();
    prod_l *= l;
    if (prod_c > n) break;
  }
  if (static_cast<int>(p.cs.size()) != static_cast<int>(ls.size()) || prod_c > n) {
    why = "N=" + std::to_string(n) + " is smaller than prod(c)";
    return CQSA_EDIVIDE;
  }
  if (n % prod_c != 0 && !(flags & CQSA_FLAG_PAD)) {
    why = "N=" + std::to_string(n) + " is not a multiple of prod(c)=" + std::to_string(prod_c) +
          " (CQSA_FLAG_PAD pads it)";
    return CQSA_EDIVIDE;
  }
  p.n_units = prod_c;
  p.unit = (n + prod_c - 1) / prod_c;
  p.n_pad = p.unit * prod_c;
  p.visits = prod_l;
  p.task_units = prod_l;
  if (p.unit * prod_l > INT32_MAX) {  // no staging of such a task exists: divide further
    why = "a task holds more than 2^31-1 tokens";
    return CQSA_EBUDGET;
  }
  return CQSA_OK;
}

// Largest plan cqsa_plan_create materializes: work items (task, unit) and mask cells.
constexpr int64_t kMaxItems = int64_t(1) << 24;
constexpr int64_t kMaxMaskCells = int64_t(1) << 32;

bool materializable(const Plan& p) {
  const int64_t tu = p.task_units;
  return p.n_units <= kMaxItems / tu && p.n_units * tu <= kMaxMaskCells / tu;
}

cqsa_status build_fixed(int64_t n, int heads, int d, cqsa_dtype dtype, const std::vector<int>& ls,
                        int64_t budget, uint32_t flags, Plan& p, std::string& why) {
  cqsa_status st = plan_shape(n, heads, d, dtype, ls, budget, flags, p, why);
  if (st != CQSA_OK) return st;
  if (!materializable(p)) {
    why = "a plan of " + std::to_string(p.n_units) + " tasks x " + std::to_string(p.task_units) +
          " units is too large to build (cqsa_plan_estimate summarizes it)";
    return CQSA_ENOMEM;
  }
  st = build_tasks(p, why);
  if (st != CQSA_OK) return st;
  build_schedule(p);
  build_descriptors(p);
  p.device_ws = align_up(p.visits * p.n * heads * int64_t(d) * 4) + align_up(p.visits * p.n * heads * int64_t(2) * 4);
  p.bwd_np = (n + 63) / 64 * 64;
  p.bwd_device_ws = bwd_layout(p).total;
  // streamed backward: the forward's mode order (device accumulators and two staging
  // sets first), restricted by the same flags; L and Delta of every row resident on the
  // device in every mode first, then kept in pinned host memory
  p.bwd_stream_fp = {false, 1, -1};
  p.bwd_host_stats = false;
  const std::pair<bool, int> bwd_order[4] = {{true, 2}, {false, 2}, {true, 1}, {false, 1}};
  for (int hs = 0; hs < 2 && p.bwd_stream_fp.bytes < 0; ++hs)
    for (const auto& m : bwd_order) {
      if ((flags & CQSA_FLAG_HOST_ACC) && m.first) continue;
      if ((flags & CQSA_FLAG_KV_SINGLE) && m.second != 1) continue;
      const int64_t bytes = bwd_stream_layout(p, m.first, m.second, hs == 1).total;
      if (fits_budget(p, bytes)) {
        p.bwd_stream_fp = {m.first, m.second, bytes};
        p.bwd_host_stats = hs == 1;
        break;
      }
    }
  return choose_mode(p, why);
}

}  // namespace

cqsa_status fallback_plan(const Plan& p, int64_t budget, Plan& out, std::string& why) {
  if (budget <= 0) {
    why = "the fallback budget must be positive";
    return CQSA_EINVAL;
  }
  // the deeper plan repeats the innermost division (an undivided plan divides with l = 3)
  std::vector<int> levels = p.ls;
  const int l = levels.back() > 1 ? levels.back() : 3;
  if (levels.size() == 1 && levels[0] == 1) levels.clear();
  std::string last_why = "no level count fits";
  cqsa_status last = CQSA_EBUDGET;
  while (static_cast<int>(levels.size()) < CQSA_MAX_LEVELS) {
    levels.push_back(l);
    int64_t prod_c = 1;
    for (int x : levels) prod_c *= x * (x - 1) + 1;
    if (prod_c > p.n) {
      why = "N=" + std::to_string(p.n) + " has fewer tokens than the " + std::to_string(prod_c) +
            " units of a deeper plan";
      return CQSA_EDIVIDE;
    }
    // padding is exact (never read), so a deeper grid that N does not divide is padded
    const uint32_t flags = (p.flags & ~CQSA_FLAG_FREE_BUDGET) | (p.n % prod_c != 0 ? CQSA_FLAG_PAD : 0u);
    std::string w;
    last = build_fixed(p.n, p.heads, p.d, p.dtype, levels, budget, flags, out, w);
    if (last == CQSA_OK) return CQSA_OK;
    last_why = w;
    if (last != CQSA_EBUDGET) break;
  }
  why = last_why;
  return last;
}

cqsa_status build_plan(int64_t n, int heads, int d, cqsa_dtype dtype, const int32_t* ls, int n_levels,
                       int64_t budget, uint32_t flags, Plan& out, std::string& why) {
  if (n < 1 || heads < 1 || (d != 64 && d != 128) || ls == nullptr || n_levels < 0 ||
      n_levels > CQSA_MAX_LEVELS || budget < 0 || (dtype != CQSA_BF16 && dtype != CQSA_F32) ||
      (flags & ~kKnownFlags) != 0) {
    why = "need n>=1, heads>=1, head_dim 64 or 128, 0<=n_levels<=" + std::to_string(CQSA_MAX_LEVELS) +
          ", budget>=0, known dtype and flags";
    return CQSA_EINVAL;
  }
  if (n > (int64_t(1) << 40) || int64_t(heads) * d > (int64_t(1) << 20)) {
    why = "problem too large";
    return CQSA_EINVAL;
  }
  if (n_levels > 0) {
    std::vector<int> levels(ls, ls + n_levels);
    for (int l : levels)
      if (l < 1 || l > CQSA_MAX_L) {
        why = "each l must be in 1..10";
        return CQSA_EINVAL;
      }
    return build_fixed(n, heads, d, dtype, levels, budget, flags, out, why);
  }
  // auto: the undivided plan first; divide (repeating l) only while the host-pinned path
  // does not fit the budget -- the out-of-memory recovery of the method
  const int l = ls[0];
  if (l < 2 || l > CQSA_MAX_L) {
    why = "auto levels need l in 2..10";
    return CQSA_EINVAL;
  }
  {
    std::string w;
    const cqsa_status st = build_fixed(n, heads, d, dtype, std::vector<int>{1}, budget, flags, out, w);
    if (st != CQSA_EBUDGET) {
      if (st != CQSA_OK) why = w;
      return st;
    }
  }
  std::vector<int> levels;
  cqsa_status last = CQSA_EBUDGET;
  std::string last_why;
  for (int k = 1; k <= CQSA_MAX_LEVELS; ++k) {
    levels.push_back(l);
    std::string w;
    last = build_fixed(n, heads, d, dtype, levels, budget, flags, out, w);
    if (last == CQSA_OK) return CQSA_OK;
    last_why = w;
    if (last == CQSA_EDIVIDE && k == 1) {
      why = w;
      return last;
    }
    if (last == CQSA_EDIVIDE) {
      why = "no level count fits the budget before N stops dividing (" + w + ")";
      return CQSA_EBUDGET;
    }
    if (last != CQSA_EBUDGET) break;
  }
  why = last_why;
  return last;
}

// ----------------------------------------------------------------------------------
// dry run: the plan's shape, footprint and traffic in closed form
// ----------------------------------------------------------------------------------
namespace {

// Upper bound of descriptor_bytes from the plan's shape alone: at most one work item per
// (task, unit) in each of the five item tables, one key run per (task, query unit, key
// unit) in each of the four run tables, and for a causal plan the largest dispatch table.
int64_t descriptor_bound(const Plan& p) {
  const int64_t items = p.n_units * p.task_units, runs = items * p.task_units;
  const int64_t order = (p.flags & CQSA_FLAG_CAUSAL) ? align_up(kMaxDispatchEntries * int64_t(sizeof(int32_t))) : 0;
  return 5 * align_up(items * int64_t(sizeof(WorkItem))) + 4 * align_up(runs * int64_t(sizeof(KeyRun))) + order;
}

// First staging mode (in cqsa_mode order, respecting the flags) whose workspace fits, by
// the budget test of cqsa_plan_create.  For a plan that cqsa_plan_create would build, the
// descriptor tables are built here when the shape bound leaves the test open, so the dry
// run and the plan agree at every budget; a larger plan is estimated with its tables off
// the device (they would have to be streamed per task, a few KiB each).
cqsa_status fit_mode(Plan& p, Footprint& fp, bool& fits, std::string& why) {
  struct Cand {
    bool dev;
    int kv;
  };
  const Cand order[4] = {{true, 2}, {false, 2}, {true, 1}, {false, 1}};
  const bool buildable = materializable(p);
  bool built = false;
  fits = false;
  for (const Cand& c : order) {
    if ((p.flags & CQSA_FLAG_HOST_ACC) && c.dev) continue;
    if ((p.flags & CQSA_FLAG_KV_SINGLE) && c.kv != 1) continue;
    const int64_t bytes = stream_layout(p, c.dev, c.kv).total;
    bool ok = p.budget == 0 || (bytes <= p.budget && (!buildable || bytes + descriptor_bound(p) <= p.budget));
    if (!ok && buildable && bytes <= p.budget) {
      if (!built) {
        const cqsa_status st = build_tasks(p, why);
        if (st != CQSA_OK) return st;
        build_descriptors(p);
        built = true;
      }
      ok = fits_budget(p, bytes);
    }
    if (ok) {
      fp = {c.dev, c.kv, bytes};
      fits = true;
      return CQSA_OK;
    }
  }
  return CQSA_OK;
}

// First streamed-backward layout in the order cqsa_plan_create tries them (L and Delta on
// the device in every staging mode first, then in pinned host memory), by fit_mode's
// budget test.
cqsa_status fit_bwd(Plan& p, Footprint& fp, bool& host_stats, bool& fits, std::string& why) {
  const std::pair<bool, int> order[4] = {{true, 2}, {false, 2}, {true, 1}, {false, 1}};
  const bool buildable = materializable(p);
  bool built = !p.tasks.empty();
  fits = false;
  for (int hs = 0; hs < 2; ++hs)
    for (const auto& m : order) {
      if ((p.flags & CQSA_FLAG_HOST_ACC) && m.first) continue;
      if ((p.flags & CQSA_FLAG_KV_SINGLE) && m.second != 1) continue;
      const int64_t bytes = bwd_stream_layout(p, m.first, m.second, hs == 1).total;
      bool ok = p.budget == 0 || (bytes <= p.budget && (!buildable || bytes + descriptor_bound(p) <= p.budget));
      if (!ok && buildable && bytes <= p.budget) {
        if (!built) {
          const cqsa_status st = build_tasks(p, why);
          if (st != CQSA_OK) return st;
          build_descriptors(p);
          built = true;
        }
        ok = fits_budget(p, bytes);
      }
      if (ok) {
        fp = {m.first, m.second, bytes};
        host_stats = hs == 1;
        fits = true;
        return CQSA_OK;
      }
    }
  return CQSA_OK;
}

int32_t mode_of(const Footprint& fp) {
  return fp.acc_on_device ? (fp.kv_buffers == 2 ? CQSA_MODE_DEVICE_ACC_KV2 : CQSA_MODE_DEVICE_ACC_KV1)
                          : (fp.kv_buffers == 2 ? CQSA_MODE_HOST_ACC_KV2 : CQSA_MODE_HOST_ACC_KV1);
}

}  // namespace

cqsa_status estimate_plan(int64_t n, int heads, int d, cqsa_dtype dtype, const int32_t* ls, int n_levels,
                          int64_t budget, uint32_t flags, const cqsa_rates& r, cqsa_estimate& out,
                          std::string& why) {
  if (n < 1 || heads < 1 || (d != 64 && d != 128) || ls == nullptr || n_levels < 0 ||
      n_levels > CQSA_MAX_LEVELS || budget < 0 || (dtype != CQSA_BF16 && dtype != CQSA_F32) ||
      (flags & ~kKnownFlags) != 0 || !(r.attn_tflops > 0) ||
      !(r.merge_gbs > 0) || !(r.h2d_gbs > 0) || !(r.d2h_gbs > 0)) {
    why = "the arguments of cqsa_plan_create, and every rate must be positive";
    return CQSA_EINVAL;
  }
  Plan p;
  Footprint fp{};
  cqsa_status st = CQSA_EBUDGET;
  if (n_levels > 0) {
    std::vector<int> levels(ls, ls + n_levels);
    for (int l : levels)
      if (l < 1 || l > CQSA_MAX_L) {
        why = "each l must be in 1..10";
        return CQSA_EINVAL;
      }
    st = plan_shape(n, heads, d, dtype, levels, budget, flags, p, why);
    bool fits = false;
    if (st == CQSA_OK) st = fit_mode(p, fp, fits, why);
    if (st != CQSA_OK) return st;
    if (!fits) {
      why = "no staging mode fits the budget";
      return CQSA_EBUDGET;
    }
  } else {
    const int l = ls[0];
    if (l < 2 || l > CQSA_MAX_L) {
      why = "auto levels need l in 2..10";
      return CQSA_EINVAL;
    }
    std::vector<int> levels{1};
    for (int k = 0; k <= CQSA_MAX_LEVELS; ++k) {
      if (k == 1) levels.clear();
      if (k >= 1) levels.push_back(l);
      std::string w;
      st = plan_shape(n, heads, d, dtype, levels, budget, flags, p, w);
      bool fits = false;
      if (st == CQSA_OK) st = fit_mode(p, fp, fits, w);
      if (st == CQSA_OK && fits) break;
      if (st == CQSA_OK) st = CQSA_EBUDGET;
      why = w.empty() ? "no level count fits the budget" : w;
      if (st != CQSA_EBUDGET) {
        if (k <= 1) return st;
        why = "no level count fits the budget before N stops dividing (" + w + ")";
        return CQSA_EBUDGET;
      }
    }
    if (st != CQSA_OK) return st;
  }
  std::memset(&out, 0, sizeof(out));
  out.n_tokens = p.n;
  out.padded_tokens = p.n_pad;
  out.heads = heads;
  out.head_dim = d;
  out.dtype = dtype;
  out.levels = static_cast<int32_t>(p.ls.size());
  for (size_t k = 0; k < p.ls.size(); ++k) {
    out.c[k] = p.cs[k];
    out.l[k] = p.ls[k];
  }
  out.n_tasks = p.n_units;
  out.unit_tokens = p.unit;
  out.visits = p.visits;
  out.task_tokens = p.task_tokens();
  out.stream_mode = fp.acc_on_device ? (fp.kv_buffers == 2 ? CQSA_MODE_DEVICE_ACC_KV2 : CQSA_MODE_DEVICE_ACC_KV1)
                                     : (fp.kv_buffers == 2 ? CQSA_MODE_HOST_ACC_KV2 : CQSA_MODE_HOST_ACC_KV1);
  out.kv_buffers = fp.kv_buffers;
  out.stream_workspace_bytes = fp.bytes;
  out.per_task_descriptor_bytes = p.task_units * int64_t(sizeof(WorkItem)) +
                                  p.task_units * p.task_units * int64_t(sizeof(KeyRun));
  const double N = double(p.n), V = double(p.visits), H = heads, D = d, e = double(p.elem_bytes());
  const int64_t row_in = p.row_in_bytes(), rowp = p.row_part_bytes();
  const bool host_acc = !fp.acc_on_device;
  out.host_pinned_bytes = 4 * p.n * row_in + p.n * heads * 4 + (host_acc ? p.n * rowp : 0);
  out.bytes_h2d = 3 * p.visits * p.n * row_in + (host_acc ? (p.visits - 1) * p.n * rowp : 0);
  if (fp.kv_buffers == 2 && !p.cs.empty()) {
    // K/V reuse between consecutive tasks of one outer task: one inner chunk each
    const int64_t c_in = p.cs.back(), l_in = p.ls.back();
    const int64_t transitions = p.n_units / c_in * (c_in - 1);
    out.bytes_d2d = c_in > 1 ? transitions * (p.task_tokens() / l_in) * row_in * 2 : 0;
    out.bytes_h2d -= out.bytes_d2d;
  }
  out.bytes_d2h = p.n * heads * int64_t(d) * p.elem_bytes() + p.n * heads * 4 +
                  (host_acc ? (p.visits - 1) * p.n * rowp : 0);
  // merge launches: a non-first visit reads accumulator + partial and writes the
  // accumulator (or, at the last visit, O and LSE); a single visit reads its partial
  const int64_t part = heads * int64_t(d + 2) * 4, fin = heads * (int64_t(d) * p.elem_bytes() + 4);
  out.merge_bytes = p.visits == 1 ? p.n * (part + fin) : p.n * ((p.visits - 2) * 3 * part + 2 * part + fin);
  out.useful_flop = (flags & CQSA_FLAG_CAUSAL) ? 2.0 * N * (N + 1) * D * H : 4.0 * N * N * D * H;
  out.t_attn_s = out.useful_flop / (r.attn_tflops * 1e12);
  out.t_merge_s = double(out.merge_bytes) / (r.merge_gbs * 1e9);
  out.t_h2d_s = double(out.bytes_h2d) / (r.h2d_gbs * 1e9);
  out.t_d2h_s = double(out.bytes_d2h) / (r.d2h_gbs * 1e9);
  const double kv_serial = fp.kv_buffers == 1 ? 2.0 * V * N * H * D * e / (r.h2d_gbs * 1e9) : 0.0;
  out.t_est_s = std::max({out.t_attn_s + out.t_merge_s + kv_serial, out.t_h2d_s, out.t_d2h_s});
  out.materializable = materializable(p) ? 1 : 0;

  // the streamed backward: at these levels, and with auto levels divided further (the
  // innermost l repeated) until one of its layouts fits
  {
    std::vector<int> levels = p.ls;
    for (;;) {
      Plan pb;
      std::string w;
      if (plan_shape(n, heads, d, dtype, levels, budget, flags, pb, w) != CQSA_OK) break;
      Footprint bf{};
      bool hs = false, fits = false;
      if (fit_bwd(pb, bf, hs, fits, w) != CQSA_OK) break;
      if (fits) {
        out.bwd_levels = static_cast<int32_t>(pb.ls.size());
        out.bwd_stream_mode = mode_of(bf);
        out.bwd_host_stats = hs ? 1 : 0;
        out.bwd_task_tokens = pb.task_tokens();
        out.bwd_stream_workspace_bytes = bf.bytes;
        break;
      }
      if (n_levels > 0 || static_cast<int>(levels.size()) >= CQSA_MAX_LEVELS) break;
      if (levels.size() == 1 && levels[0] == 1) levels.clear();
      levels.push_back(ls[0]);
    }
    if (out.bwd_levels == 0) out.bwd_stream_workspace_bytes = -1;
  }
  return CQSA_OK;
}

}  // namespace cqsa
