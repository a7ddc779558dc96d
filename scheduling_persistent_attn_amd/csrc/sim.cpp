// Schedule simulator: the backward DAG of the DASH technical summary
// (section 2.1: compute and reduction phases as nodes; data dependencies and
// the mandatory accumulation order as edges; critical-path length as the
// objective; each KV tile's work an unbroken chain on one unit) with the
// depth condition of Lemma 1 (section 2.2 B) checked on every order edge.
//
// Events per task: S, E, R, F.  Weights: S->E = c (c_diag on a causal
// diagonal tile), R->F = r, all other edges 0.  Order edges F(rank q) ->
// R(rank q+1) per dQ tile are the zero-weight edges that Lemma 1 adds.  The replay
// advances workers in time order (and decides the dynamic dispatch); the DAG
// pass computes longest paths in topological order, with and without the
// order edges.

#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <queue>
#include <vector>

#include "../../include/dash_attn.h"
#include "schedule.h"
#include "table.h"

namespace {

struct SimTask {
  int group, g, i, j, rank, item;
};

struct Problem {
  int mask, schedule, N, G, groups, P;
  double c, c_diag, r;
  std::vector<SimTask> tasks;       // global dispatch order
  std::vector<int> item_first;      // first task of each item (+ sentinel)
  std::vector<int> order_prev;      // task of rank-1 in the same dQ tile, or -1
  std::vector<int> order_next;      // task of rank+1, or -1
  double cost(int t) const {
    const SimTask& k = tasks[t];
    return (mask == dash::MASK_CAUSAL && k.i == k.j) ? c_diag : c;
  }
};

bool build(Problem& pb, const dash::GroupTable& tb) {
  const int ipg = (int)tb.offs.size() - 1;
  const int items = ipg * pb.groups;
  const int per = (int)tb.tasks.size();
  pb.item_first.assign(items + 1, 0);
  pb.tasks.reserve((size_t)per * pb.groups);
  for (int grp = 0; grp < pb.groups; ++grp) {
    for (int it = 0; it < ipg; ++it) {
      pb.item_first[grp * ipg + it] = (int)pb.tasks.size();
      for (int s = tb.offs[it]; s < tb.offs[it + 1]; ++s) {
        const dash::TableTask& t = tb.tasks[s];
        pb.tasks.push_back({grp, t.g, t.i, t.j, t.rank, grp * ipg + it});
      }
    }
  }
  pb.item_first[items] = (int)pb.tasks.size();
  // slot of (group, g, j, rank) -> task
  const long long tiles = (long long)pb.groups * pb.G * pb.N;
  std::vector<int> base(tiles + 1, 0);
  for (long long x = 0; x < tiles; ++x) {
    const int j = (int)(x % pb.N);
    base[x + 1] = base[x] + dash::contributors(pb.mask, pb.N, j);
  }
  std::vector<int> slot(base[tiles], -1);
  for (int t = 0; t < (int)pb.tasks.size(); ++t) {
    const SimTask& k = pb.tasks[t];
    const long long x = ((long long)k.group * pb.G + k.g) * pb.N + k.j;
    const int n = base[x + 1] - base[x];
    if (k.rank < 0 || k.rank >= n || slot[base[x] + k.rank] != -1) return false;
    slot[base[x] + k.rank] = t;
  }
  pb.order_prev.assign(pb.tasks.size(), -1);
  pb.order_next.assign(pb.tasks.size(), -1);
  for (long long x = 0; x < tiles; ++x) {
    for (int q = base[x] + 1; q < base[x + 1]; ++q) {
      pb.order_prev[slot[q]] = slot[q - 1];
      pb.order_next[slot[q - 1]] = slot[q];
    }
  }
  return true;
}

// Timed replay.  Fills assign[item] and returns false on a stall.
bool replay(const Problem& pb, int dispatch, std::vector<int>& assign, double* makespan) {
  const int items = (int)pb.item_first.size() - 1;
  const int ntask = (int)pb.tasks.size();
  assign.assign(items, -1);
  std::vector<double> F(ntask, -1.0);
  std::vector<int> waiter(ntask, -1);        // task waiting for F of this task
  std::vector<double> waiter_E(ntask, 0.0);
  std::vector<int> wk_item(pb.P, -1), wk_pos(pb.P, 0), wk_last(pb.P, -1);
  typedef std::pair<double, int> Ev;
  std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> heap;
  int next_item = 0;
  int done = 0;
  double mk = 0.0;
  for (int w = 0; w < pb.P; ++w) heap.push(Ev(0.0, w));

  auto take = [&](int w) -> bool {
    int k;
    if (dispatch == 0) {
      k = wk_last[w] < 0 ? w : wk_last[w] + pb.P;
    } else {
      k = next_item++;
    }
    if (k >= items) return false;
    wk_last[w] = k;
    wk_item[w] = k;
    wk_pos[w] = 0;
    assign[k] = w;
    return true;
  };

  // finish task t of worker w with reduction start Rt; wakes a chain of waiters
  std::function<void(int, int, double)> finish = [&](int w, int t, double Rt) {
    std::vector<std::pair<int, double>> stack;  // (task, Rt)
    std::vector<int> who;
    stack.push_back({t, Rt});
    who.push_back(w);
    while (!stack.empty()) {
      const int tt = stack.back().first;
      const double rt = stack.back().second;
      const int ww = who.back();
      stack.pop_back();
      who.pop_back();
      const double f = rt + pb.r;
      F[tt] = f;
      mk = std::max(mk, f);
      ++done;
      if (++wk_pos[ww] >= pb.item_first[wk_item[ww] + 1] - pb.item_first[wk_item[ww]])
        wk_item[ww] = -1;
      heap.push(Ev(f, ww));
      const int nx = pb.order_next[tt];
      if (nx >= 0 && waiter[nx] >= 0) {
        const int w2 = waiter[nx];
        waiter[nx] = -1;
        stack.push_back({nx, std::max(waiter_E[nx], f)});
        who.push_back(w2);
      }
    }
  };

  while (!heap.empty()) {
    const Ev ev = heap.top();
    heap.pop();
    const int w = ev.second;
    if (wk_item[w] < 0 && !take(w)) continue;
    const int t = pb.item_first[wk_item[w]] + wk_pos[w];
    const double E = ev.first + pb.cost(t);
    const int pr = pb.order_prev[t];
    if (pr < 0) {
      finish(w, t, E);
    } else if (F[pr] >= 0.0) {
      finish(w, t, std::max(E, F[pr]));
    } else {
      waiter[t] = w;
      waiter_E[t] = E;
    }
  }
  *makespan = mk;
  return done == ntask;
}

// Longest path over the event graph; returns false on a cycle.
bool longest(const Problem& pb, const std::vector<int>& assign, bool with_order,
             std::vector<double>& depth) {
  const int ntask = (int)pb.tasks.size();
  const int items = (int)pb.item_first.size() - 1;
  const int nn = 4 * ntask;
  // successor lists in CSR form
  std::vector<int> deg(nn + 1, 0);
  std::vector<std::pair<int, int>> edges;  // (u, v), weights from node kinds
  edges.reserve((size_t)ntask * 6);
  for (int t = 0; t < ntask; ++t) {
    edges.push_back({4 * t + 0, 4 * t + 1});
    edges.push_back({4 * t + 1, 4 * t + 2});
    edges.push_back({4 * t + 2, 4 * t + 3});
  }
  for (int k = 0; k < items; ++k)
    for (int t = pb.item_first[k]; t + 1 < pb.item_first[k + 1]; ++t)
      edges.push_back({4 * t + 3, 4 * (t + 1)});
  std::vector<int> last_item(pb.P, -1);
  for (int k = 0; k < items; ++k) {
    const int w = assign[k];
    if (w < 0) continue;
    if (last_item[w] >= 0)
      edges.push_back({4 * (pb.item_first[last_item[w] + 1] - 1) + 3, 4 * pb.item_first[k]});
    last_item[w] = k;
  }
  if (with_order)
    for (int t = 0; t < ntask; ++t)
      if (pb.order_prev[t] >= 0) edges.push_back({4 * pb.order_prev[t] + 3, 4 * t + 2});
  for (auto& e : edges) deg[e.first + 1]++;
  for (int x = 0; x < nn; ++x) deg[x + 1] += deg[x];
  std::vector<int> adj(edges.size());
  std::vector<int> fill(deg.begin(), deg.end() - 1);
  std::vector<int> indeg(nn, 0);
  for (auto& e : edges) {
    adj[fill[e.first]++] = e.second;
    indeg[e.second]++;
  }
  depth.assign(nn, 0.0);
  std::vector<int> ready;
  for (int x = 0; x < nn; ++x)
    if (indeg[x] == 0) ready.push_back(x);
  int seen = 0;
  while (!ready.empty()) {
    const int u = ready.back();
    ready.pop_back();
    ++seen;
    const int kind = u & 3;
    const double wgt = kind == 0 ? pb.cost(u >> 2) : (kind == 2 ? pb.r : 0.0);
    for (int e = deg[u]; e < deg[u + 1]; ++e) {
      const int v = adj[e];
      if (depth[u] + wgt > depth[v]) depth[v] = depth[u] + wgt;
      if (--indeg[v] == 0) ready.push_back(v);
    }
  }
  return seen == nn;
}

}  // namespace

namespace {

// Simulation of any schedule given as a table (closed forms included).
int run_problem(Problem& pb, const dash::GroupTable& tb, int dispatch, dash_sim_result* out) {
  if (!build(pb, tb)) return DASH_ERR_TABLE;
  // workers beyond the items stay idle under either dispatch: keep no state
  // for them (item k runs on worker k either way)
  pb.P = std::min(pb.P, std::max(1, (int)pb.item_first.size() - 1));
  const int P = pb.P;
  std::vector<int> assign;
  double replay_mk = 0.0;
  const bool ok = replay(pb, dispatch, assign, &replay_mk);
  const int items = (int)pb.item_first.size() - 1;
  if (!ok) {
    for (int k = 0; k < items; ++k) assign[k] = k % P;
  }
  std::vector<double> d_base, d_full;
  longest(pb, assign, false, d_base);
  const bool acyclic = longest(pb, assign, true, d_full);

  dash_sim_result res;
  res.total_work = 0.0;
  for (int t = 0; t < (int)pb.tasks.size(); ++t) res.total_work += pb.cost(t) + pb.r;
  res.base_makespan = 0.0;
  for (double x : d_base) res.base_makespan = std::max(res.base_makespan, x);
  res.deadlock = (!ok || !acyclic) ? 1 : 0;
  if (!acyclic) {
    res.makespan = INFINITY;
  } else {
    res.makespan = 0.0;
    for (double x : d_full) res.makespan = std::max(res.makespan, x);
  }
  res.order_edges = 0;
  res.violations = 0;
  res.max_deficit = 0.0;
  for (int t = 0; t < (int)pb.tasks.size(); ++t) {
    const int pr = pb.order_prev[t];
    if (pr < 0) continue;
    res.order_edges++;
    const double deficit = d_base[4 * pr + 3] - d_base[4 * t + 2];
    if (deficit > 0.0) {
      res.violations++;
      res.max_deficit = std::max(res.max_deficit, deficit);
    }
  }
  const int used = std::min(P, items);
  res.efficiency = (res.makespan > 0.0 && std::isfinite(res.makespan))
                       ? res.total_work / ((double)used * res.makespan)
                       : 0.0;
  *out = res;
  return DASH_OK;
}


}  // namespace

extern "C" int dash_sim_run(int mask, int schedule, int N, int G, int groups, int P,
                            int dispatch, double c_full, double c_diag, double r,
                            dash_sim_result* out) {
  if (!out) return DASH_ERR_NULL;
  if (N < 1 || G < 1 || groups < 1 || P < 1 || (dispatch != 0 && dispatch != 1))
    return DASH_ERR_SHAPE;
  if (dash_schedule_num_items(mask, schedule, N) < 0) return DASH_ERR_SCHEDULE_MASK;
  if (!(c_full >= 0.0) || !(c_diag >= 0.0) || !(r >= 0.0)) return DASH_ERR_SHAPE;
  const double tasks_est = (double)groups * G * N * (double)N;
  if (tasks_est > 2.0e7) return DASH_ERR_UNSUPPORTED;
  Problem pb;
  pb.mask = mask;
  pb.schedule = schedule;
  pb.N = N;
  pb.G = G;
  pb.groups = groups;
  pb.P = P;
  pb.c = c_full;
  pb.c_diag = c_diag;
  pb.r = r;
  const int st = run_problem(pb, dash::closed_form_table(mask, schedule, N, G), dispatch, out);
  return st == DASH_ERR_TABLE ? DASH_ERR_SCHEDULE_MASK : st;
}

// The deterministic schedule with the shortest critical path for a shape and
// worker count: every candidate that applies to the mask and tile count is
// simulated, deadlocked ones are skipped, and ties go to the earlier
// candidate of {SYMMETRIC_SHIFT, SHIFT, DESCENDING_Q, NAIVE}.
extern "C" int dash_sim_select(int mask, int N, int G, int groups, int P, int dispatch,
                               double c_full, double c_diag, double r, int* schedule,
                               dash_sim_result* out) {
  if (!schedule) return DASH_ERR_NULL;
  static const int order[4] = {DASH_SCHED_SYMMETRIC_SHIFT, DASH_SCHED_SHIFT,
                               DASH_SCHED_DESCENDING_Q, DASH_SCHED_NAIVE};
  int best = -1;
  dash_sim_result best_res = {};
  for (int s : order) {
    if (s == DASH_SCHED_SYMMETRIC_SHIFT && (mask != DASH_MASK_CAUSAL || N % 2 != 0)) continue;
    dash_sim_result res;
    const int st = dash_sim_run(mask, s, N, G, groups, P, dispatch, c_full, c_diag, r, &res);
    if (st != DASH_OK) return st;
    if (res.deadlock) continue;
    if (best < 0 || res.makespan < best_res.makespan) {
      best = s;
      best_res = res;
    }
  }
  if (best < 0) return DASH_ERR_UNSUPPORTED;
  *schedule = best;
  if (out) *out = best_res;
  return DASH_OK;
}

namespace dash {

int sim_table(int mask, int N, int G, int groups, int P, int dispatch, double c_full, double c_diag, double r,
              const GroupTable& t, dash_sim_result* out) {
  if (!out) return DASH_ERR_NULL;
  if (N < 1 || G < 1 || groups < 1 || P < 1 || (dispatch != 0 && dispatch != 1)) return DASH_ERR_SHAPE;
  if (mask != MASK_FULL && mask != MASK_CAUSAL) return DASH_ERR_SCHEDULE_MASK;
  if (!(c_full >= 0.0) || !(c_diag >= 0.0) || !(r >= 0.0)) return DASH_ERR_SHAPE;
  if ((double)groups * (double)t.tasks.size() > 2.0e7) return DASH_ERR_UNSUPPORTED;
  Problem pb;
  pb.mask = mask;
  pb.schedule = -1;
  pb.N = N;
  pb.G = G;
  pb.groups = groups;
  pb.P = P;
  pb.c = c_full;
  pb.c_diag = c_diag;
  pb.r = r;
  return run_problem(pb, t, dispatch, out);
}

}  // namespace dash
