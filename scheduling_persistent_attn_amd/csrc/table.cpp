// Task tables: checks against the kernels' hand-off protocol, the closed-form
// schedules written out as tables, and a search over a family of block-wise
// lockstep walks that contains the closed forms (DASH technical summary,
// section 2: the schedule that minimises the backward DAG's critical path,
// chosen per shape and hardware; section 2.1: one key/value tile's work is
// an unbroken chain on one unit).
//
// Deadlock freedom.  A persistent workgroup takes items in dispatch order
// and never gives one back, and every dQ hand-off waits on the previous rank.
// The kernels pipeline each hand-off over the passes that follow it: within
// one key/value tile's run, the turn of pass n is taken at the end of pass
// n+1 and the slice is published in pass n+3, after the turn of pass n+1 was
// taken; the run's last pass drains everything before the tile changes.  So
// a table is safe on P workgroups when
//   (1) the waits-for graph of those events -- each run's event sequence plus
//       "published by rank q-1" -> "turn taken by rank q" for every pass of
//       every dQ tile -- has no cycle, and
//   (2) the items split into consecutive dispatch blocks of at most P items
//       such that no item waits on an item of a later block.
// Proof sketch: take the earliest block with unfinished work.  Items of later
// blocks are dispatched only after all of its items, and earlier blocks are
// done; if one of its items is not yet dispatched, fewer than P workgroups
// hold items and an idle one takes it; if all are dispatched, the earliest
// unfinished event of the acyclic graph has all of its predecessors done and
// its workgroup can take it.  Either way the launch progresses.

#include "table.h"

#include <stdint.h>

#include <algorithm>
#include <tuple>
#include <vector>

#include "schedule.h"

namespace dash {

// Largest table the host checks accept: tasks per group, and tasks x passes
// for the event graph.
constexpr long long kMaxTableTasks = 1LL << 24;
constexpr long long kMaxTableEvents = 1LL << 24;

long long table_tiles(int mask, int N) {
  return mask == MASK_CAUSAL ? (long long)N * (N + 1) / 2 : (long long)N * N;
}

namespace {

// First slot of dQ tile (g, j) among one group's slots (one per contributor;
// the slot of a rank, or of a contributing key/value tile i, is base + it:
// the contributors of j are KV tiles 0 .. n_j - 1).
struct TileSlots {
  int N;
  std::vector<long long> base;
  TileSlots(int mask, int N_, int G) : N(N_), base((size_t)G * N_ + 1, 0) {
    for (long long x = 0; x < (long long)G * N; ++x)
      base[x + 1] = base[x] + contributors(mask, N, (int)(x % N));
  }
  long long at(int g, int j) const { return base[(size_t)g * N + j]; }
};

}  // namespace

int table_validate(int mask, int N, int G, int items, const int* offs, const int* tasks, GroupTable* out,
                   std::vector<uint32_t>* packed) {
  if (!offs || !tasks) return DASH_ERR_NULL;
  if (mask != MASK_FULL && mask != MASK_CAUSAL) return DASH_ERR_SCHEDULE_MASK;
  if (N < 1 || N >= (1 << 14) || G < 1 || G >= (1 << 16)) return DASH_ERR_SHAPE;
  const long long n = (long long)G * table_tiles(mask, N);
  if (n > kMaxTableTasks) return DASH_ERR_UNSUPPORTED;
  // every item holds at least one run (of a key/value tile, or in the
  // per-head form of one head's key/value tile)
  if (items < 1 || (long long)items > (long long)G * N) return DASH_ERR_TABLE;
  if (offs[0] != 0 || offs[items] != n) return DASH_ERR_TABLE;
  for (int k = 0; k < items; ++k)
    if (offs[k + 1] <= offs[k]) return DASH_ERR_TABLE;
  // each (g, j) slot filled by exactly one rank and one key/value tile: with
  // n tasks for n slots this is exact coverage
  TileSlots ts(mask, N, G);
  std::vector<char> rank_seen((size_t)n, 0), kv_seen((size_t)n, 0);
  for (long long t = 0; t < n; ++t) {
    const int g = tasks[4 * t], i = tasks[4 * t + 1], j = tasks[4 * t + 2], r = tasks[4 * t + 3];
    if (g < 0 || g >= G || i < 0 || i >= N || j < 0 || j >= N) return DASH_ERR_TABLE;
    if (mask == MASK_CAUSAL && j < i) return DASH_ERR_TABLE;
    if (r < 0 || r >= contributors(mask, N, j)) return DASH_ERR_TABLE;
    const long long b = ts.at(g, j);
    if (rank_seen[b + r] || kv_seen[b + i]) return DASH_ERR_TABLE;
    rank_seen[b + r] = 1;
    kv_seen[b + i] = 1;
  }
  // runs: one contiguous run per key/value tile (all its heads and query
  // tiles), or else one per (head, key/value tile)
  bool tile_form = true, head_form = true;
  {
    std::vector<char> tile_run(N, 0), head_run((size_t)G * N, 0);
    for (int k = 0; k < items; ++k) {
      int prev_i = -1, prev_gi = -1;
      for (int t = offs[k]; t < offs[k + 1]; ++t) {
        const int g = tasks[4 * t], i = tasks[4 * t + 1], gi = g * N + i;
        if (i != prev_i) {
          if (tile_run[i]) tile_form = false;
          tile_run[i] = 1;
          prev_i = i;
        }
        if (gi != prev_gi) {
          if (head_run[gi]) head_form = false;
          head_run[gi] = 1;
          prev_gi = gi;
        }
      }
    }
  }
  if (!tile_form && !head_form) return DASH_ERR_TABLE;
  const bool split = !tile_form;
  if (out) {
    out->offs.assign(offs, offs + items + 1);
    out->tasks.resize((size_t)n);
    for (long long t = 0; t < n; ++t)
      out->tasks[t] = {tasks[4 * t], tasks[4 * t + 1], tasks[4 * t + 2], tasks[4 * t + 3]};
    out->split = split;
  }
  if (packed) {
    packed->resize((size_t)n * 2);
    auto run_key = [&](long long t) { return split ? tasks[4 * t] * N + tasks[4 * t + 1] : tasks[4 * t + 1]; };
    for (int k = 0; k < items; ++k) {
      for (int t = offs[k]; t < offs[k + 1]; ++t) {
        const int i = tasks[4 * t + 1];
        const uint32_t begin = t == offs[k] || run_key(t - 1) != run_key(t);
        const uint32_t end = t == offs[k + 1] - 1 || run_key(t + 1) != run_key(t);
        (*packed)[2 * t] = (uint32_t)i | ((uint32_t)tasks[4 * t + 2] << 16);
        (*packed)[2 * t + 1] =
            (uint32_t)tasks[4 * t] | ((uint32_t)tasks[4 * t + 3] << 16) | (begin << 30) | (end << 31);
      }
    }
  }
  return DASH_OK;
}

int table_protocol(int mask, int N, const GroupTable& tb, int passes, int P, int* blocks, int* widest) {
  const int items = (int)tb.offs.size() - 1;
  const long long n = (long long)tb.tasks.size();
  const long long tiles = table_tiles(mask, N);
  if (items < 1 || n == 0 || n % tiles != 0 || passes < 1 || P < 1) return DASH_ERR_TABLE;
  if (n * passes > kMaxTableEvents) return DASH_ERR_UNSUPPORTED;
  const int G = (int)(n / tiles);
  TileSlots ts(mask, N, G);
  std::vector<int> slot((size_t)n, -1), owner((size_t)n, 0);
  for (int k = 0; k < items; ++k)
    for (int t = tb.offs[k]; t < tb.offs[k + 1]; ++t) owner[t] = k;
  for (long long t = 0; t < n; ++t) {
    const TableTask& x = tb.tasks[t];
    slot[ts.at(x.g, x.j) + x.rank] = (int)t;
  }
  auto pred = [&](long long t) {
    const TableTask& x = tb.tasks[t];
    return x.rank > 0 ? slot[ts.at(x.g, x.j) + x.rank - 1] : -1;
  };
  auto succ = [&](long long t) {
    const TableTask& x = tb.tasks[t];
    return x.rank + 1 < contributors(mask, N, x.j) ? slot[ts.at(x.g, x.j) + x.rank + 1] : -1;
  };

  // (2) dispatch blocks: an item and every later item it waits on share one
  int nb = 0, wid = 0;
  {
    std::vector<int> reach(items);
    for (int k = 0; k < items; ++k) {
      int m = k;
      for (int t = tb.offs[k]; t < tb.offs[k + 1]; ++t) {
        const int pr = pred(t);
        if (pr >= 0) m = std::max(m, owner[pr]);
      }
      reach[k] = m;
    }
    int start = 0, end = 0;
    for (int k = 0; k < items; ++k) {
      end = std::max(end, reach[k]);
      if (k == end) {
        ++nb;
        wid = std::max(wid, k - start + 1);
        start = k + 1;
      }
    }
  }
  if (blocks) *blocks = nb;
  if (widest) *widest = wid;
  if (wid > P) return DASH_ERR_TABLE;

  // (1) the waits-for graph of turn-taken (A) and published (R) events.
  // Node 2 * (t * passes + p) + 0 is A of pass p of task t, + 1 its R.
  const long long nodes = 2 * n * passes;
  std::vector<int> next((size_t)nodes, -1), indeg((size_t)nodes, 0);
  auto A = [&](long long t, int p) { return (int)(2 * (t * passes + p)); };
  auto R = [&](long long t, int p) { return (int)(2 * (t * passes + p) + 1); };
  for (int k = 0; k < items; ++k) {
    int last = -1;  // the previous run's final event
    auto link = [&](int u) {
      if (last >= 0) {
        next[last] = u;
        indeg[u]++;
      }
      last = u;
    };
    int t0 = tb.offs[k];
    while (t0 < tb.offs[k + 1]) {
      int t1 = t0;
      while (t1 + 1 < tb.offs[k + 1] && same_run(tb, (size_t)t1)) ++t1;
      // passes 0 .. L of the run; pass m takes the turn of m-1 at its end
      // and publishes m-3 in its body; the drain publishes the rest
      const long long L = (long long)(t1 - t0 + 1) * passes - 1;
      auto ev = [&](long long m, bool pub) {
        const long long t = t0 + m / passes;
        const int p = (int)(m % passes);
        return pub ? R(t, p) : A(t, p);
      };
      for (long long m = 1; m <= L; ++m) {
        if (m >= 3) link(ev(m - 3, true));
        link(ev(m - 1, false));
      }
      if (L >= 2) link(ev(L - 2, true));
      if (L >= 1) link(ev(L - 1, true));
      link(ev(L, false));
      link(ev(L, true));
      t0 = t1 + 1;
    }
  }
  for (long long t = 0; t < n; ++t)
    if (pred(t) >= 0)
      for (int p = 0; p < passes; ++p) indeg[A(t, p)]++;
  std::vector<int> ready;
  ready.reserve(1024);
  for (long long u = 0; u < nodes; ++u)
    if (indeg[u] == 0) ready.push_back((int)u);
  long long seen = 0;
  auto drop = [&](int v) {
    if (--indeg[v] == 0) ready.push_back(v);
  };
  while (!ready.empty()) {
    const int u = ready.back();
    ready.pop_back();
    ++seen;
    if (next[u] >= 0) drop(next[u]);
    if (u & 1) {
      const long long t = (u >> 1) / passes;
      const int p = (int)((u >> 1) % passes);
      const int s = succ(t);
      if (s >= 0) drop(A(s, p));
    }
  }
  return seen == nodes ? DASH_OK : DASH_ERR_TABLE;
}

GroupTable closed_form_table(int mask, int schedule, int N, int G) {
  GroupTable tb;
  const int ipg = items_per_group(mask, schedule, N);
  tb.offs.push_back(0);
  for (int it = 0; it < ipg; ++it) {
    const int len = item_len(mask, schedule, N, G, it);
    for (int s = 0; s < len; ++s) {
      const Task t = task_at(mask, schedule, N, G, it, s);
      tb.tasks.push_back({t.g, t.i, t.j, t.rank});
    }
    tb.offs.push_back((int)tb.tasks.size());
  }
  return tb;
}

// Passes per task of the kernel that runs tiles of T keys at head dim D
// (one pass = the rows of a query tile that the workgroup's waves cover
// together: 32 rows when the waves split the head dim, else 64).
int passes_per_task(int T, int D) {
  if (T == 256) return D == 128 ? 8 : 4;  // 32-row passes at D = 128, 64-row at 64
  const int NW = T / 32, DB = D / 32;
  return T / (32 * (NW / DB));
}

namespace {

// Single-head walk of one unit of the family: a key/value chain, or a
// symmetric pair (causal, even N): (i, j) per step.
std::vector<std::pair<int, int>> unit_walk(int mask, int N, int kind, int u) {
  std::vector<std::pair<int, int>> w;
  const int first = mask == MASK_CAUSAL ? u : 0;
  switch (kind) {
    case DASH_FAMILY_SYMMETRIC: {
      const int h = N / 2, p = u;
      for (int s = 0; s < h; ++s) w.push_back({p, h + (p + s) % h});
      for (int j = p; j < h; ++j) w.push_back({p, j});
      for (int j = N - 1; j >= N - 1 - p; --j) w.push_back({N - 1 - p, j});
      break;
    }
    case DASH_FAMILY_SHIFT:
      if (mask == MASK_CAUSAL) {
        for (int j = u; j < N; ++j) w.push_back({u, j});
      } else {
        for (int s = 0; s < N; ++s) w.push_back({u, (u + s) % N});
      }
      break;
    case DASH_FAMILY_DESCENDING:
      for (int j = N - 1; j >= first; --j) w.push_back({u, j});
      break;
    default:  // DASH_FAMILY_ASCENDING
      for (int j = first; j < N; ++j) w.push_back({u, j});
      break;
  }
  return w;
}

}  // namespace

bool family_applies(int mask, int N, int kind) {
  switch (kind) {
    case DASH_FAMILY_SYMMETRIC: return mask == MASK_CAUSAL && N % 2 == 0;
    case DASH_FAMILY_SHIFT:
    case DASH_FAMILY_DESCENDING:
    case DASH_FAMILY_PACKED: return true;
    case DASH_FAMILY_ASCENDING: return mask == MASK_FULL;  // causal: the shift walk
    default: return false;
  }
}

namespace {

// The packed family: every (head, key/value tile) chain on its own -- the
// shift walk of that tile (causal: the diagonal upward; full: cyclic from
// the diagonal) -- packed longest first into `bins` items, each chain to the
// least loaded bin (lower index on ties); non-empty bins in index order are
// the items.  A task's no-wait start is its position in its item (the items
// start together, one per workgroup), and dQ tile (g, j) is reduced in the
// order (position, item).  Every wait then points to an earlier position,
// or to the same position in an earlier item, so the order has no cycle.
// With grouped heads the chains of one key/value tile land in different
// items: the per-head form.
GroupTable packed_table(int mask, int N, int G, int bins) {
  struct Chain {
    int len, g, i;
  };
  std::vector<Chain> chains;
  chains.reserve((size_t)G * N);
  for (int g = 0; g < G; ++g)
    for (int i = 0; i < N; ++i) chains.push_back({mask == MASK_CAUSAL ? N - i : N, g, i});
  std::stable_sort(chains.begin(), chains.end(), [](const Chain& a, const Chain& b) {
    return a.len != b.len ? a.len > b.len : (a.g != b.g ? a.g < b.g : a.i < b.i);
  });
  std::vector<long long> load(bins, 0);
  std::vector<std::vector<int>> bin_chains(bins);
  for (int c = 0; c < (int)chains.size(); ++c) {
    int b = 0;
    for (int x = 1; x < bins; ++x)
      if (load[x] < load[b]) b = x;
    bin_chains[b].push_back(c);
    load[b] += chains[c].len;
  }
  GroupTable tb;
  tb.offs.push_back(0);
  std::vector<int> pos;  // position of each task in its item
  for (int b = 0; b < bins; ++b) {
    if (bin_chains[b].empty()) continue;
    int at = 0;
    for (int c : bin_chains[b]) {
      const Chain& ch = chains[c];
      for (int s = 0; s < ch.len; ++s) {
        const int j = mask == MASK_CAUSAL ? ch.i + s : (ch.i + s) % N;
        tb.tasks.push_back({ch.g, ch.i, j, 0});
        pos.push_back(at++);
      }
    }
    tb.offs.push_back((int)tb.tasks.size());
  }
  // the form: whole-tile when each key/value tile's chains happen to form
  // one run (always with one head), else per-head
  {
    std::vector<char> seen(N, 0);
    bool tile_form = true;
    for (size_t k = 0; k + 1 < tb.offs.size() && tile_form; ++k)
      for (int t = tb.offs[k]; t < tb.offs[k + 1]; ++t)
        if (t == tb.offs[k] || tb.tasks[t].i != tb.tasks[t - 1].i) {
          if (seen[tb.tasks[t].i]) {
            tile_form = false;
            break;
          }
          seen[tb.tasks[t].i] = 1;
        }
    tb.split = !tile_form;
  }
  // ranks: (position, item) order per dQ tile
  const int items = (int)tb.offs.size() - 1;
  std::vector<std::vector<std::tuple<int, int, int>>> at((size_t)G * N);
  for (int k = 0; k < items; ++k)
    for (int t = tb.offs[k]; t < tb.offs[k + 1]; ++t)
      at[(size_t)tb.tasks[t].g * N + tb.tasks[t].j].push_back({pos[t], k, t});
  for (auto& v : at) {
    std::sort(v.begin(), v.end());
    for (int r = 0; r < (int)v.size(); ++r) tb.tasks[std::get<2>(v[r])].rank = r;
  }
  return tb;
}

}  // namespace

int packed_bins(int N, int G, int groups, int P) {
  const long long chains = (long long)G * N;
  const long long b = groups >= 1 ? P / groups : P;
  return (int)std::max(1LL, std::min(chains, b));
}

// The family's table: units (chains, or symmetric pairs) in ascending or
// descending order, grouped into dispatch blocks of `block` consecutive
// units; each unit walks its query tiles step by step, every step taken for
// all G heads in turn; dQ tile (g, j) is reduced in the order (block, step
// at which the unit reaches j, unit position) -- lockstep arrival inside a
// block, blocks one after another.
GroupTable family_table(int mask, int N, int G, int kind, int order, int block) {
  // more bins than chains leave the extra ones empty: the same table
  if (kind == DASH_FAMILY_PACKED) return packed_table(mask, N, G, std::max(1, std::min(block, G * N)));
  const int units = kind == DASH_FAMILY_SYMMETRIC ? N / 2 : N;
  std::vector<std::vector<std::pair<int, int>>> walks(units);
  std::vector<int> unit_of(units);
  for (int pos = 0; pos < units; ++pos) {
    unit_of[pos] = order == 0 ? pos : units - 1 - pos;
    walks[pos] = unit_walk(mask, N, kind, unit_of[pos]);
  }
  // arrival keys per query tile, then single-head ranks per (unit, step)
  std::vector<std::vector<std::tuple<int, int, int>>> at(N);
  for (int pos = 0; pos < units; ++pos)
    for (int s = 0; s < (int)walks[pos].size(); ++s) at[walks[pos][s].second].push_back({pos / block, s, pos});
  std::vector<std::vector<int>> rank(units);
  for (int pos = 0; pos < units; ++pos) rank[pos].assign(walks[pos].size(), 0);
  for (int j = 0; j < N; ++j) {
    std::sort(at[j].begin(), at[j].end());
    for (int r = 0; r < (int)at[j].size(); ++r) rank[std::get<2>(at[j][r])][std::get<1>(at[j][r])] = r;
  }
  GroupTable tb;
  tb.offs.push_back(0);
  for (int pos = 0; pos < units; ++pos) {
    for (int s = 0; s < (int)walks[pos].size(); ++s)
      for (int g = 0; g < G; ++g) tb.tasks.push_back({g, walks[pos][s].first, walks[pos][s].second, rank[pos][s]});
    tb.offs.push_back((int)tb.tasks.size());
  }
  return tb;
}

// Block sizes tried for a family: the widest that P allows, half of it, and
// one unit per block, largest first.
std::vector<int> family_blocks(int units, int P) {
  const int m = std::min(units, P);
  std::vector<int> out = {m};
  if (m / 2 >= 1 && m / 2 != m) out.push_back(m / 2);
  if (out.back() != 1) out.push_back(1);
  return out;
}

}  // namespace dash

namespace {

void write_table(const dash::GroupTable& tb, int* items, int* offs, int* tasks) {
  *items = (int)tb.offs.size() - 1;
  for (size_t k = 0; k < tb.offs.size(); ++k) offs[k] = tb.offs[k];
  for (size_t t = 0; t < tb.tasks.size(); ++t) {
    tasks[4 * t] = tb.tasks[t].g;
    tasks[4 * t + 1] = tb.tasks[t].i;
    tasks[4 * t + 2] = tb.tasks[t].j;
    tasks[4 * t + 3] = tb.tasks[t].rank;
  }
}

}  // namespace

extern "C" {

long long dash_schedule_table_tasks(int mask, int N, int G) {
  if ((mask != 0 && mask != 1) || N < 1 || G < 1) return -1;
  return (long long)G * dash::table_tiles(mask, N);
}

int dash_schedule_table_closed_form(int mask, int schedule, int N, int G, int* items, int* item_offsets,
                                    int* tasks) {
  if (!items || !item_offsets || !tasks) return DASH_ERR_NULL;
  if (G < 1 || N < 1) return DASH_ERR_SHAPE;
  if (schedule == DASH_SCHED_ATOMIC || dash_schedule_num_items(mask, schedule, N) < 0)
    return DASH_ERR_SCHEDULE_MASK;
  if ((long long)G * dash::table_tiles(mask, N) > dash::kMaxTableTasks) return DASH_ERR_UNSUPPORTED;
  write_table(dash::closed_form_table(mask, schedule, N, G), items, item_offsets, tasks);
  return DASH_OK;
}

int dash_schedule_table_family(int mask, int N, int G, int kind, int order, int block, int* items,
                               int* item_offsets, int* tasks) {
  if (!items || !item_offsets || !tasks) return DASH_ERR_NULL;
  if (mask != DASH_MASK_FULL && mask != DASH_MASK_CAUSAL) return DASH_ERR_SCHEDULE_MASK;
  if (N < 1 || G < 1 || block < 1 || (order != 0 && order != 1)) return DASH_ERR_SHAPE;
  if (kind == DASH_FAMILY_PACKED && order != 0) return DASH_ERR_SHAPE;  // one order only
  if (!dash::family_applies(mask, N, kind)) return DASH_ERR_SCHEDULE_MASK;
  if ((long long)G * dash::table_tiles(mask, N) > dash::kMaxTableTasks) return DASH_ERR_UNSUPPORTED;
  write_table(dash::family_table(mask, N, G, kind, order, block), items, item_offsets, tasks);
  return DASH_OK;
}

int dash_schedule_table_check(int S, int D, int mask, int G, int P, int items, const int* item_offsets,
                              const int* tasks) {
  const int T = dash_attn_tile_size(S, D);
  if (T == 0) return DASH_ERR_UNSUPPORTED;
  if (S < 1 || P < 1) return DASH_ERR_SHAPE;
  const int N = (S + T - 1) / T;
  dash::GroupTable tb;
  int st = dash::table_validate(mask, N, G, items, item_offsets, tasks, &tb, nullptr);
  if (st != DASH_OK) return st;
  // per-head runs need the 256-key tile kernels' fp32 partial dK/dV
  if (tb.split && T != 256) return DASH_ERR_UNSUPPORTED;
  return dash::table_protocol(mask, N, tb, dash::passes_per_task(T, D), P, nullptr, nullptr);
}

size_t dash_schedule_table_pack(int S, int D, int mask, int G, int items, const int* item_offsets,
                                const int* tasks, void* out, size_t out_bytes, int* status) {
  int dummy = 0;
  int* st_out = status ? status : &dummy;
  const int T = dash_attn_tile_size(S, D);
  if (T == 0) {
    *st_out = DASH_ERR_UNSUPPORTED;
    return 0;
  }
  if (S < 1) {
    *st_out = DASH_ERR_SHAPE;
    return 0;
  }
  const int N = (S + T - 1) / T;
  dash::GroupTable tb;
  std::vector<uint32_t> words;
  int st = dash::table_validate(mask, N, G, items, item_offsets, tasks, &tb, &words);
  if (st == DASH_OK && tb.split && T != 256) st = DASH_ERR_UNSUPPORTED;
  int widest = 0;
  const int passes = dash::passes_per_task(T, D);
  // any grid at least as wide as the widest block: checked by the kernels
  if (st == DASH_OK) st = dash::table_protocol(mask, N, tb, passes, 1 << 30, nullptr, &widest);
  if (st != DASH_OK) {
    *st_out = st;
    return 0;
  }
  const size_t n = tb.tasks.size();
  const size_t bytes = ((size_t)dash::table_task_words(items) + 2 * n) * sizeof(uint32_t);
  *st_out = DASH_OK;
  if (!out) return bytes;
  if (out_bytes < bytes) {
    *st_out = DASH_ERR_WORKSPACE;
    return bytes;
  }
  uint32_t* w = (uint32_t*)out;
  const uint32_t form = tb.split ? dash::kTableSplit : 0u;
  const uint32_t hdr[dash::kTableHeaderWords] = {dash::kTableMagic, (uint32_t)N, (uint32_t)G, (uint32_t)mask | form,
                                                 (uint32_t)passes, (uint32_t)items, (uint32_t)widest,
                                                 (uint32_t)n};
  for (int x = 0; x < dash::kTableHeaderWords; ++x) w[x] = hdr[x];
  const int tw = dash::table_task_words(items);
  for (int x = dash::kTableHeaderWords; x < tw; ++x) {
    const int k = x - dash::kTableHeaderWords;
    w[x] = k <= items ? (uint32_t)item_offsets[k] : 0u;
  }
  for (size_t x = 0; x < 2 * n; ++x) w[tw + x] = words[x];
  return bytes;
}

int dash_sim_table(int mask, int N, int G, int groups, int P, int dispatch, double c_full, double c_diag,
                   double r, int items, const int* item_offsets, const int* tasks, dash_sim_result* out) {
  if (!out) return DASH_ERR_NULL;
  dash::GroupTable tb;
  const int st = dash::table_validate(mask, N, G, items, item_offsets, tasks, &tb, nullptr);
  if (st != DASH_OK) return st;
  return dash::sim_table(mask, N, G, groups, P, dispatch, c_full, c_diag, r, tb, out);
}

int dash_schedule_search(int S, int D, int mask, int G, int groups, int P, double c_full, double c_diag, double r,
                         int* items, int* item_offsets, int* tasks, int* family, dash_sim_result* out) {
  if (!items || !item_offsets || !tasks) return DASH_ERR_NULL;
  const int T = dash_attn_tile_size(S, D);
  if (T == 0) return DASH_ERR_UNSUPPORTED;
  if (S < 1 || G < 1 || groups < 1 || P < 1) return DASH_ERR_SHAPE;
  if (mask != DASH_MASK_FULL && mask != DASH_MASK_CAUSAL) return DASH_ERR_SCHEDULE_MASK;
  if (!(c_full >= 0.0) || !(c_diag >= 0.0) || !(r >= 0.0)) return DASH_ERR_SHAPE;
  const int N = (S + T - 1) / T;
  if ((long long)G * dash::table_tiles(mask, N) > dash::kMaxTableTasks) return DASH_ERR_UNSUPPORTED;
  const int passes = dash::passes_per_task(T, D);
  static const int kinds[5] = {DASH_FAMILY_SYMMETRIC, DASH_FAMILY_SHIFT, DASH_FAMILY_DESCENDING,
                               DASH_FAMILY_ASCENDING, DASH_FAMILY_PACKED};
  bool found = false;
  dash::GroupTable best;
  dash_sim_result best_res = {};
  int best_fam[3] = {0, 0, 0};
  for (int kind : kinds) {
    if (!dash::family_applies(mask, N, kind)) continue;
    // per-head tables run on the 256-key tile kernels only
    if (kind == DASH_FAMILY_PACKED && G > 1 && T != 256) continue;
    const bool packed = kind == DASH_FAMILY_PACKED;
    const int units = kind == DASH_FAMILY_SYMMETRIC ? N / 2 : N;
    const std::vector<int> blocks =
        packed ? std::vector<int>{dash::packed_bins(N, G, groups, P)} : dash::family_blocks(units, P);
    for (int order = 0; order < (packed ? 1 : 2); ++order) {
      for (int b : blocks) {
        dash::GroupTable tb = dash::family_table(mask, N, G, kind, order, b);
        int st = dash::table_protocol(mask, N, tb, passes, P, nullptr, nullptr);
        if (st == DASH_ERR_TABLE) continue;
        if (st != DASH_OK) return st;
        dash_sim_result res;
        st = dash::sim_table(mask, N, G, groups, P, 1, c_full, c_diag, r, tb, &res);
        if (st != DASH_OK) return st;
        if (res.deadlock) continue;
        if (!found || res.makespan < best_res.makespan) {
          found = true;
          best = std::move(tb);
          best_res = res;
          best_fam[0] = kind;
          best_fam[1] = order;
          best_fam[2] = b;
        }
      }
    }
  }
  if (!found) return DASH_ERR_UNSUPPORTED;
  write_table(best, items, item_offsets, tasks);
  if (family) {
    family[0] = best_fam[0];
    family[1] = best_fam[1];
    family[2] = best_fam[2];
  }
  if (out) *out = best_res;
  return DASH_OK;
}

}  // extern "C"
