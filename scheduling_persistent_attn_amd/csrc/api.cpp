// C ABI of libdash_attn.so: argument checks, workspace layout, launches.
// See include/dash_attn.h for the contract of every entry point.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/dash_attn.h"
#include "kernels.h"
#include "schedule.h"

namespace {

constexpr int kMaxDevices = 64;

// wall-clock limit of one turn wait, in microseconds (dash_attn_set_watchdog)
std::atomic<long long> g_watchdog_us{2000000};

struct DeviceInfo {
  bool ready = false;
  int cus = 0;
  long long wall_khz = 0;
  int bpc[2][2][2] = {};  // [D==128][T==128][causal] resident blocks per CU
  int bpc_wide[2][2] = {};  // [D==128][causal] of the 256-key tile kernels
};

DeviceInfo g_dev[kMaxDevices];
std::mutex g_mu;

int device_info(DeviceInfo** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DASH_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.ready) {
    int cus = 0, khz = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return DASH_ERR_HIP;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
      khz = 100000;
    d.cus = cus;
    d.wall_khz = khz;
    // the 64- and 128-key tile kernels (larger problems use the 256-key tiles)
    const int cfgs[2][2] = {{64, 64}, {128, 128}};
    for (auto& cfg : cfgs)
      for (int causal = 0; causal < 2; ++causal)
        d.bpc[cfg[0] == 128][cfg[1] == 128][causal] =
            dash::bwd_blocks_per_cu(cfg[0], cfg[1], causal != 0);
    for (int causal = 0; causal < 2; ++causal) {
      d.bpc_wide[1][causal] = dash::bwd_wide_blocks_per_cu(causal != 0);
      d.bpc_wide[0][causal] = dash::bwd_wide64_blocks_per_cu(causal != 0);
    }
    d.ready = true;
  }
  *out = &d;
  return DASH_OK;
}

inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Persistent workgroups the backward kernel for tile T runs per compute unit.
int blocks_per_cu(const DeviceInfo& d, int D, int T, int mask) {
  if (T == 256) return d.bpc_wide[D == 128][mask];
  return d.bpc[D == 128][T == 128][mask];
}

// Turn counters per dQ tile: one per slice a wave reduces per pass -- 32 rows
// x 32 features for tiles of 64 and 128, 32 rows x 16 features for 256.
int slices_per_tile(int T, int D) { return T == 256 ? T * D / 512 : T * D / 1024; }

struct Layout {
  int T = 0, N = 0, NW = 0, parts = 1;
  size_t ctrl = 0, waits = 0, counters = 0, delta = 0, lse2 = 0, dqacc = 0, dkvp = 0, table = 0, trace = 0,
         total = 0;
  size_t table_bytes = 0;
  long long n_counters = 0, n_rows = 0, n_dqacc = 0, n_dkvp = 0, n_trace = 0;
};

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Pure argument checks (no device access).
int check_shape(int B, int Hq, int Hkv, int S, int D, int mask, int schedule) {
  if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0) return DASH_ERR_SHAPE;
  if (Hq % Hkv != 0) return DASH_ERR_SHAPE;
  if (D != 64 && D != 128) return DASH_ERR_UNSUPPORTED;
  if (mask != DASH_MASK_FULL && mask != DASH_MASK_CAUSAL) return DASH_ERR_SCHEDULE_MASK;
  if ((schedule < DASH_SCHED_NAIVE || schedule > DASH_SCHED_AUTO) && schedule != DASH_SCHED_TABLE)
    return DASH_ERR_SCHEDULE_MASK;
  return DASH_OK;
}

// A launch with fewer items than this leaves compute units of an MI355X idle
// (256 compute units; the 256-key tile kernel runs one workgroup on each).
constexpr int kSplitTargetItems = 256;

// Query-head parts per base item, a function of the shape alone: with 256-key
// tiles and grouped heads, the smallest divisor d of G for which the launch
// has at least kSplitTargetItems items, else G; 1 otherwise.  For AUTO, the
// largest over the schedules it can resolve to (the workspace then covers
// any of them).
int head_parts(int B, int Hkv, int G, int N, int T, int mask, int schedule) {
  if (T != 256 || G == 1 || N == 0) return 1;
  // a table in the per-head form writes one fp32 partial per query head
  // (a whole-tile table leaves that buffer unused)
  if (schedule == DASH_SCHED_TABLE) return G;
  if (schedule == DASH_SCHED_AUTO) {
    int m = 1;
    for (int s = DASH_SCHED_NAIVE; s <= DASH_SCHED_SYMMETRIC_SHIFT; ++s) {
      if (s == DASH_SCHED_SYMMETRIC_SHIFT && (mask != DASH_MASK_CAUSAL || N % 2 != 0)) continue;
      const int d = head_parts(B, Hkv, G, N, T, mask, s);
      m = d > m ? d : m;
    }
    return m;
  }
  const long long base = (long long)B * Hkv * dash::items_per_group(mask, schedule, N);
  for (int d = 1; d <= G; ++d)
    if (G % d == 0 && base * d >= kSplitTargetItems) return d;
  return G;
}

// Trace records per item: its longest task list.
int trace_len(int mask, int schedule, int N, int Gp) {
  return Gp * (dash::paired_items(mask, schedule, N) ? N + 1 : N);
}

int make_layout(int B, int Hq, int Hkv, int S, int D, int mask, int schedule, Layout* L) {
  L->T = dash_attn_tile_size(S, D);
  if (L->T == 0) return DASH_ERR_UNSUPPORTED;
  L->N = (S + L->T - 1) / L->T;
  L->parts = head_parts(B, Hkv, Hq / Hkv, L->N, L->T, mask, schedule);
  L->NW = slices_per_tile(L->T, D);
  const long long rows = (long long)B * Hq * L->N * L->T;
  L->n_rows = rows;
  L->n_counters = (long long)B * Hq * L->N * L->NW;
  L->n_dqacc = rows * D;
  // every element offset the kernels form must fit in 32 bits
  const long long elems = (long long)B * S * Hq * D;
  if (elems >= (1LL << 31) || L->n_dqacc >= (1LL << 31)) return DASH_ERR_UNSUPPORTED;
  size_t off = 0;
  L->ctrl = off;
  off += round256(64 * sizeof(int));
  // the kernel finds the wait counters right after the 64 control words
  static_assert(64 * sizeof(int) % 256 == 0, "wait counters follow ctrl directly");
  L->waits = off;
  off += round256((size_t)dash::kWaitSlots * 4 * sizeof(unsigned long long));
  L->counters = off;
  off += round256((size_t)L->n_counters * sizeof(int));
  L->delta = off;
  off += round256((size_t)rows * sizeof(float));
  L->lse2 = off;
  off += round256((size_t)rows * sizeof(float));
  L->dqacc = off;
  off += round256((size_t)L->n_dqacc * sizeof(float));
  // last, so that no other offset depends on the number of parts
  L->dkvp = off;
  L->n_dkvp = L->parts > 1 ? 2LL * B * Hkv * L->parts * L->N * L->T * D : 0;
  off += round256((size_t)L->n_dkvp * sizeof(float));
  // AUTO: room for the searched table's device form, which the prepare phase
  // copies in when AUTO resolves to it (the largest table of this shape).
  // TABLE reserves it too, so that AUTO resolved to a table keeps every
  // offset (the debug build's trace follows it).
  L->table = off;
  if (schedule == DASH_SCHED_AUTO || schedule == DASH_SCHED_TABLE) {
    const int G = Hq / Hkv;
    const long long n = dash_schedule_table_tasks(mask, L->N, G);
    L->table_bytes = ((size_t)dash::table_task_words(G * L->N) + 2 * (size_t)(n > 0 ? n : 0)) * sizeof(unsigned);
    off += round256(L->table_bytes);
  }
#ifdef DASH_TASK_TRACE
  // the debug build's task trace: 64 bytes per (item, step), for the
  // longest item of any schedule the call could run
  L->trace = off;
  L->n_trace = 0;
  for (int s = DASH_SCHED_NAIVE; s <= DASH_SCHED_ATOMIC; ++s) {
    if (schedule != DASH_SCHED_AUTO && s != schedule) continue;
    if (s == DASH_SCHED_SYMMETRIC_SHIFT && (mask != DASH_MASK_CAUSAL || L->N % 2 != 0)) continue;
    const int parts = head_parts(B, Hkv, Hq / Hkv, L->N, L->T, mask, s);
    const long long items = (long long)B * Hkv * parts * dash::items_per_group(mask, s, L->N);
    const long long n = items * trace_len(mask, s, L->N, Hq / Hkv / parts);
    L->n_trace = n > L->n_trace ? n : L->n_trace;
  }
  // a table schedule (also the searched table AUTO may resolve to): one
  // record per task
  if (schedule == DASH_SCHED_TABLE || schedule == DASH_SCHED_AUTO) {
    const long long n = (long long)B * Hq * L->N * L->N;
    L->n_trace = n > L->n_trace ? n : L->n_trace;
  }
  off += round256((size_t)L->n_trace * 64);
#endif
  L->total = off;
  return DASH_OK;
}

// Weights of the schedule simulator for DASH_SCHED_AUTO, per task: a full
// tile and a causal diagonal tile cost the same in this kernel (the diagonal
// is computed whole and masked), and the part of a dQ hand-off that stays
// exposed is about a tenth of a task (it is pipelined behind later passes).
constexpr double kAutoC = 1.0, kAutoCDiag = 1.0, kAutoR = 0.1;

// AUTO considers the searched table only up to this many simulated tasks
// (groups x tasks per group), so that its first call stays within about two
// seconds of host time.
constexpr long long kAutoTableSimTasks = 1LL << 18;

// The choice of DASH_SCHED_AUTO on a device with `grid` persistent
// workgroups, host only.  Every deterministic closed form that applies, each
// with its own split of the query heads (a split group simulates as `parts`
// groups of G/parts heads, in the same dispatch order), and with
// `allow_table` the library's searched table (dash_schedule_search with the
// same weights) where its workspace is the closed forms' (no head split on
// 64/128-key tiles or with G = 1, else the closed forms already reserve G
// partial slots).  The shortest critical path wins; ties go to the earlier
// of SYMMETRIC_SHIFT, SHIFT, DESCENDING_Q, NAIVE, then the table.  With the
// table chosen, `packed` receives its device form and `items` its items.
int auto_decide(int B, int Hq, int Hkv, int S, int D, int mask, int grid, bool allow_table, int* out,
                std::vector<unsigned char>* packed, int* items) {
  int st = check_shape(B, Hq, Hkv, S, D, mask, DASH_SCHED_NAIVE);
  if (st != DASH_OK) return st;
  Layout L;
  st = make_layout(B, Hq, Hkv, S, D, mask, DASH_SCHED_NAIVE, &L);
  if (st != DASH_OK) return st;
  if (B == 0 || S == 0) {
    *out = DASH_SCHED_NAIVE;
    return DASH_OK;
  }
  if (grid <= 0) return DASH_ERR_SHAPE;
  const int G = Hq / Hkv;
  int sched = -1;
  double best = 0.0;
  {
    static const int order[4] = {DASH_SCHED_SYMMETRIC_SHIFT, DASH_SCHED_SHIFT, DASH_SCHED_DESCENDING_Q,
                                 DASH_SCHED_NAIVE};
    st = DASH_OK;
    for (int s : order) {
      if (s == DASH_SCHED_SYMMETRIC_SHIFT && (mask != DASH_MASK_CAUSAL || L.N % 2 != 0)) continue;
      const int parts = head_parts(B, Hkv, G, L.N, L.T, mask, s);
      dash_sim_result res;
      const int rs = dash_sim_run(mask, s, L.N, G / parts, B * Hkv * parts, grid, 1, kAutoC, kAutoCDiag,
                                  kAutoR, &res);
      if (rs != DASH_OK) {
        st = rs;
        break;
      }
      if (res.deadlock) continue;
      if (sched < 0 || res.makespan < best) {
        sched = s;
        best = res.makespan;
      }
    }
    if (st == DASH_OK && sched < 0) st = DASH_ERR_UNSUPPORTED;
  }
  if (st == DASH_ERR_UNSUPPORTED || st == DASH_ERR_SCHEDULE_MASK) {
    // too large to simulate: the simulator's usual order on co-resident
    // groups, else the descending order (causal) or the naive one
    const bool sym_ok = mask == DASH_MASK_CAUSAL && L.N % 2 == 0 &&
                        dash::items_per_group(mask, DASH_SCHED_SYMMETRIC_SHIFT, L.N) <= grid;
    const bool shift_ok = dash::items_per_group(mask, DASH_SCHED_SHIFT, L.N) <= grid;
    *out = sym_ok ? DASH_SCHED_SYMMETRIC_SHIFT
                  : shift_ok ? DASH_SCHED_SHIFT
                             : mask == DASH_MASK_CAUSAL ? DASH_SCHED_DESCENDING_Q : DASH_SCHED_NAIVE;
    return DASH_OK;
  }
  if (st != DASH_OK) return st;
  *out = sched;
  const long long per_group = dash_schedule_table_tasks(mask, L.N, G);
  const bool same_workspace =
      L.T != 256 || G == 1 || head_parts(B, Hkv, G, L.N, L.T, mask, DASH_SCHED_AUTO) == G;
  if (!allow_table || !same_workspace || per_group <= 0 || per_group * B * Hkv > kAutoTableSimTasks)
    return DASH_OK;
  std::vector<int> offs((size_t)G * L.N + 1), tasks((size_t)per_group * 4);
  int n_items = 0;
  dash_sim_result res;
  st = dash_schedule_search(S, D, mask, G, B * Hkv, grid, kAutoC, kAutoCDiag, kAutoR, &n_items, offs.data(),
                            tasks.data(), nullptr, &res);
  // no candidate runs on this grid, or none beats the closed forms
  if (st != DASH_OK || res.deadlock || !(res.makespan < best)) return DASH_OK;
  int pst = DASH_OK;
  const size_t bytes =
      dash_schedule_table_pack(S, D, mask, G, n_items, offs.data(), tasks.data(), nullptr, 0, &pst);
  // the AUTO layout's table region holds the largest table of the shape
  Layout LA;
  if (pst != DASH_OK || make_layout(B, Hq, Hkv, S, D, mask, DASH_SCHED_AUTO, &LA) != DASH_OK ||
      bytes > LA.table_bytes)
    return DASH_OK;
  packed->resize(bytes);
  dash_schedule_table_pack(S, D, mask, G, n_items, offs.data(), tasks.data(), packed->data(), bytes, &pst);
  if (pst != DASH_OK) return DASH_OK;
  *items = n_items;
  *out = DASH_SCHED_TABLE;
  return DASH_OK;
}

// AUTO's resolution for a shape on a device: the schedule, and for the
// searched table its device form in pinned host memory (held until the
// process ends), copied into the workspace by every prepare phase.
struct AutoChoice {
  int schedule = DASH_SCHED_NAIVE;
  const void* table = nullptr;
  size_t table_bytes = 0;
  int items = 0;
};

struct AutoEntry {
  int dev, B, Hq, Hkv, S, D, mask;
  bool allow_table;
  AutoChoice choice;
};
std::vector<AutoEntry> g_auto;
std::mutex g_auto_mu;

// Resolves DASH_SCHED_AUTO for a shape on the current device (cached).
int auto_schedule(int B, int Hq, int Hkv, int S, int D, int mask, bool allow_table, AutoChoice* out) {
  int st = check_shape(B, Hq, Hkv, S, D, mask, DASH_SCHED_NAIVE);
  if (st != DASH_OK) return st;
  if (B == 0 || S == 0) {
    *out = AutoChoice();
    return DASH_OK;
  }
  DeviceInfo* dev = nullptr;
  st = device_info(&dev);
  if (st != DASH_OK) return st;
  int dev_id = 0;
  if (hipGetDevice(&dev_id) != hipSuccess) return DASH_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_auto_mu);
  for (const AutoEntry& e : g_auto)
    if (e.dev == dev_id && e.B == B && e.Hq == Hq && e.Hkv == Hkv && e.S == S && e.D == D &&
        e.mask == mask && e.allow_table == allow_table) {
      *out = e.choice;
      return DASH_OK;
    }
  const int T = dash_attn_tile_size(S, D);
  const int grid = dev->cus * blocks_per_cu(*dev, D, T, mask);
  if (grid <= 0) return DASH_ERR_HIP;
  AutoChoice c;
  std::vector<unsigned char> packed;
  st = auto_decide(B, Hq, Hkv, S, D, mask, grid, allow_table, &c.schedule, &packed, &c.items);
  if (st != DASH_OK) return st;
  if (c.schedule == DASH_SCHED_TABLE) {
    void* host = nullptr;
    if (hipHostMalloc(&host, packed.size(), hipHostMallocDefault) != hipSuccess) return DASH_ERR_HIP;
    std::memcpy(host, packed.data(), packed.size());
    c.table = host;
    c.table_bytes = packed.size();
  }
  g_auto.push_back({dev_id, B, Hq, Hkv, S, D, mask, allow_table, c});
  *out = c;
  return DASH_OK;
}

}  // namespace

extern "C" {

int dash_attn_bwd_auto_schedule(int B, int Hq, int Hkv, int S, int D, int mask) {
  AutoChoice c;
  const int st = auto_schedule(B, Hq, Hkv, S, D, mask, true, &c);
  return st == DASH_OK ? c.schedule : -st;
}

int dash_attn_bwd_auto_schedule_on(int B, int Hq, int Hkv, int S, int D, int mask, int grid) {
  int sched = 0, items = 0;
  std::vector<unsigned char> packed;
  const int st = auto_decide(B, Hq, Hkv, S, D, mask, grid, true, &sched, &packed, &items);
  return st == DASH_OK ? sched : -st;
}

int dash_attn_bwd_head_parts(int B, int Hq, int Hkv, int S, int D, int mask, int schedule) {
  if (check_shape(B, Hq, Hkv, S, D, mask, schedule) != DASH_OK) return 0;
  Layout L;
  if (make_layout(B, Hq, Hkv, S, D, mask, schedule, &L) != DASH_OK) return 0;
  return L.parts;
}

int dash_attn_tile_size(int S, int D) {
  if (D == 64) return S <= 512 ? 64 : 256;
  if (D == 128) return S <= 512 ? 128 : 256;
  return 0;
}

size_t dash_attn_bwd_workspace_size(int B, int Hq, int Hkv, int S, int D, int mask,
                                    int schedule) {
  if (check_shape(B, Hq, Hkv, S, D, mask, schedule) != DASH_OK) return 0;
  Layout L;
  if (make_layout(B, Hq, Hkv, S, D, mask, schedule, &L) != DASH_OK) return 0;
  return L.total;
}

const char* dash_status_string(int status) {
  switch (status) {
    case DASH_OK: return "ok";
    case DASH_ERR_NULL: return "a required pointer is NULL";
    case DASH_ERR_SHAPE: return "invalid shape or misaligned pointer";
    case DASH_ERR_UNSUPPORTED: return "unsupported head dim, size or schedule residency";
    case DASH_ERR_SCHEDULE_MASK: return "invalid mask/schedule combination";
    case DASH_ERR_WORKSPACE: return "workspace missing or too small";
    case DASH_ERR_HIP: return "HIP runtime error";
    case DASH_ERR_TIMEOUT: return "device watchdog fired in an ordered reduction";
    case DASH_ERR_NOT_PREPARED: return "backward run on a workspace not prepared since the last run";
    case DASH_ERR_TABLE: return "task table invalid, could deadlock, or refused by the kernel";
    default: return "unknown status";
  }
}

int dash_attn_bwd_grid_size(int S, int D, int mask) {
  const int T = dash_attn_tile_size(S, D);
  if (T == 0 || (mask != 0 && mask != 1)) return 0;
  DeviceInfo* d = nullptr;
  if (device_info(&d) != DASH_OK) return 0;
  return d->cus * blocks_per_cu(*d, D, T, mask);
}

int dash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int Hq, int Hkv, int S, int D, int mask, void* stream) {
  int st = check_shape(B, Hq, Hkv, S, D, mask, DASH_SCHED_NAIVE);
  if (st != DASH_OK) return st;
  // 32-bit element offsets inside the kernel; the batch is a grid dimension
  if ((long long)B * S * Hq * D >= (1LL << 31) || B > 65535) return DASH_ERR_UNSUPPORTED;
  if (B == 0 || S == 0) return DASH_OK;
  if (!q || !k || !v || !o || !lse) return DASH_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return DASH_ERR_SHAPE;
  dash::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.S = S;
  p.G = Hq / Hkv;
  p.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  if (dash::launch_fwd(D, mask == DASH_MASK_CAUSAL, p, (hipStream_t)stream) != hipSuccess)
    return DASH_ERR_HIP;
  return DASH_OK;
}

}  // extern "C"

namespace {

// A table schedule's launch arguments (already checked by the caller).
struct TableArgs {
  const void* table;
  int items;
  int grid;  // workgroups to launch at most; 0 = the device's persistent grid
};

// Everything a backward launch needs, checked once.
struct BwdPlan {
  Layout L;
  int grid = 0;
  // AUTO resolved to the searched table: its pinned host copy, copied into
  // the workspace's table region by the prepare phase
  const void* upload_src = nullptr;
  void* upload_dst = nullptr;
  size_t upload_bytes = 0;
  dash::PreParams pp;
  dash::BwdParams bp;
  dash::FinParams fp;
  dash::DkvFinParams kp;
};

// Validates the arguments of a backward and fills the launch parameters.
// Sets *empty for B == 0 or S == 0 (nothing to launch).  The pointers that a
// phase does not use may be NULL: `need` selects which are required
// (1 = preprocess inputs, 2 = main-kernel inputs and outputs).
int plan_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S,
             int D, int mask, int schedule, void* workspace, size_t workspace_bytes, int need,
             BwdPlan* P, bool* empty, const TableArgs* tab = nullptr, bool allow_table = true) {
  *empty = false;
  int st = check_shape(B, Hq, Hkv, S, D, mask, schedule);
  if (st != DASH_OK) return st;
  Layout& L = P->L;
  st = make_layout(B, Hq, Hkv, S, D, mask, schedule, &L);
  if (st != DASH_OK) return st;
  if (schedule == DASH_SCHED_SYMMETRIC_SHIFT && (mask != DASH_MASK_CAUSAL || (L.N % 2) != 0))
    return DASH_ERR_SCHEDULE_MASK;
  // the main phase of a table schedule needs its table
  if (schedule == DASH_SCHED_TABLE && (need & 2) && !tab) return DASH_ERR_SCHEDULE_MASK;
  if (B == 0 || S == 0) {
    *empty = true;
    return DASH_OK;
  }
  if ((need & 1) && (!o || !dout || !lse)) return DASH_ERR_NULL;
  if ((need & 2) && (!q || !k || !v || !dout || !dq || !dk || !dv)) return DASH_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return DASH_ERR_SHAPE;
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256))
    return DASH_ERR_WORKSPACE;

  TableArgs auto_tab;
  if (schedule == DASH_SCHED_AUTO) {
    AutoChoice c;
    st = auto_schedule(B, Hq, Hkv, S, D, mask, allow_table, &c);
    if (st != DASH_OK) return st;
    schedule = c.schedule;
    const size_t table_off = L.table;
    // the resolved schedule's layout: the same offsets, at most as many parts
    // (a searched table is chosen only where it has as many as AUTO)
    st = make_layout(B, Hq, Hkv, S, D, mask, schedule, &L);
    if (st != DASH_OK) return st;
    if (schedule == DASH_SCHED_TABLE) {
      auto_tab = {(char*)workspace + table_off, c.items, 0};
      tab = &auto_tab;
      P->upload_src = c.table;
      P->upload_dst = (char*)workspace + table_off;
      P->upload_bytes = c.table_bytes;
    }
  }
  DeviceInfo* dev = nullptr;
  st = device_info(&dev);
  if (st != DASH_OK) return st;
  int grid = dev->cus * blocks_per_cu(*dev, D, L.T, mask);
  if (grid <= 0) return DASH_ERR_HIP;
  const int G = Hq / Hkv;
  const int base_items = tab ? tab->items : dash::items_per_group(mask, schedule, L.N);
  // a table's items are its own; the closed forms repeat theirs per part
  const int ipg = tab ? base_items : base_items * L.parts;
  if (tab && tab->grid > 0) grid = tab->grid;
  // The shift family waits on chains that come later in the dispatch order,
  // so the items of one part of a group must be able to run at once.
  if ((schedule == DASH_SCHED_SHIFT || schedule == DASH_SCHED_SYMMETRIC_SHIFT) && base_items > grid)
    return DASH_ERR_UNSUPPORTED;

  char* ws = (char*)workspace;
  dash::PreParams& pp = P->pp;
  pp.o = o;
  pp.dout = dout;
  pp.lse = lse;
  pp.delta = (float*)(ws + L.delta);
  pp.lse2 = (float*)(ws + L.lse2);
  pp.counters = (int*)(ws + L.counters);
  pp.ctrl = (int*)(ws + L.ctrl);
  pp.waits = (unsigned long long*)(ws + L.waits);
  pp.dqacc = (float*)(ws + L.dqacc);
  pp.n_counters = L.n_counters;
  pp.n_dqacc = L.n_dqacc;
  pp.zero_dqacc = schedule == DASH_SCHED_ATOMIC;
  pp.inv_scale = (float)__builtin_sqrt((double)D);
  pp.B = B;
  pp.Hq = Hq;
  pp.S = S;
  pp.D = D;
  pp.NT = L.N * L.T;

  dash::BwdParams& bp = P->bp;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.dout = dout;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.delta = pp.delta;
  bp.lse2 = pp.lse2;
  bp.dqacc = pp.dqacc;
  bp.counters = pp.counters;
  bp.ctrl = pp.ctrl;
  bp.B = B;
  bp.Hq = Hq;
  bp.Hkv = Hkv;
  bp.S = S;
  bp.N = L.N;
  bp.G = G;
  bp.mask = mask;
  bp.schedule = schedule;
  bp.items_per_group = ipg;
  bp.total_items = B * Hkv * ipg;
  bp.parts = L.parts;
  bp.Gp = tab ? G : G / L.parts;
  bp.base_items = base_items;
  bp.dkv_part = L.parts > 1 ? (float*)(ws + L.dkvp) : nullptr;
  bp.NT = L.N * L.T;
  bp.table = tab ? (const unsigned*)tab->table : nullptr;
  bp.table_tasks = tab ? (int)dash_schedule_table_tasks(mask, L.N, G) : 0;
#ifdef DASH_TASK_TRACE
  bp.trace = (unsigned long long*)(ws + L.trace);
  bp.trace_len = trace_len(mask, schedule, L.N, bp.Gp);
#else
  bp.trace = nullptr;
  bp.trace_len = 0;
#endif
  bp.scale = (float)(1.0 / __builtin_sqrt((double)D));
  bp.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  bp.spin_ticks = g_watchdog_us.load() * dev->wall_khz / 1000;
  P->grid = grid < bp.total_items ? grid : bp.total_items;

  dash::DkvFinParams& kp = P->kp;
  kp.dkv_part = bp.dkv_part;
  kp.dk = dk;
  kp.dv = dv;
  kp.ctrl = pp.ctrl;
  kp.B = B;
  kp.Hkv = Hkv;
  kp.S = S;
  kp.NT = bp.NT;
  kp.D = D;
  kp.parts = L.parts;
  // a table's partials exist only when its kernel marked them (per-head form)
  kp.need_mark = tab ? 1 : 0;
  kp.scale = (float)(1.0 / __builtin_sqrt((double)D));

  dash::FinParams& fp = P->fp;
  fp.dqacc = pp.dqacc;
  fp.ctrl = pp.ctrl;
  fp.dq = dq;
  fp.B = B;
  fp.Hq = Hq;
  fp.S = S;
  fp.N = L.N;
  fp.scale = bp.scale;
  return DASH_OK;
}

// The prepare phase: the preprocess, and the searched table's copy into the
// workspace when AUTO resolved to it (from pinned host memory, so the copy is
// asynchronous and may be captured).
int launch_prepare(const BwdPlan& P, hipStream_t s) {
  if (dash::launch_preprocess(P.pp, s) != hipSuccess) return DASH_ERR_HIP;
  if (P.upload_bytes &&
      hipMemcpyAsync(P.upload_dst, P.upload_src, P.upload_bytes, hipMemcpyHostToDevice, s) != hipSuccess)
    return DASH_ERR_HIP;
  return DASH_OK;
}

int launch_main_phase(const BwdPlan& P, int D, int mask, hipStream_t s) {
  const bool causal = mask == DASH_MASK_CAUSAL;
  if (P.L.T == 256) {
    const bool d128 = D == 128;
    if ((d128 ? dash::launch_bwd_wide(causal, P.bp, P.grid, s) : dash::launch_bwd_wide64(causal, P.bp, P.grid, s)) !=
        hipSuccess)
      return DASH_ERR_HIP;
    if (P.bp.schedule == DASH_SCHED_ATOMIC &&
        (d128 ? dash::launch_finalize_wide(P.fp, s) : dash::launch_finalize_wide64(P.fp, s)) != hipSuccess)
      return DASH_ERR_HIP;
    if (P.L.parts > 1 && dash::launch_dkv_finalize(P.kp, s) != hipSuccess) return DASH_ERR_HIP;
    return DASH_OK;
  }
  if (dash::launch_bwd_main(D, P.L.T, causal, P.bp, P.grid, s) != hipSuccess) return DASH_ERR_HIP;
  if (P.bp.schedule == DASH_SCHED_ATOMIC &&
      dash::launch_finalize_atomic(D, P.L.T, P.fp, s) != hipSuccess)
    return DASH_ERR_HIP;
  return DASH_OK;
}

// dash_attn_bwd_table (phases 3: preprocess and main phase) and its run
// phase alone (2, after dash_attn_bwd_prepare with DASH_SCHED_TABLE).
int table_phases(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S, int D,
                 int mask, const void* table, size_t table_bytes, int items, int grid, void* workspace,
                 size_t workspace_bytes, void* stream, int phases) {
  int st = check_shape(B, Hq, Hkv, S, D, mask, DASH_SCHED_TABLE);
  if (st != DASH_OK) return st;
  if (B == 0 || S == 0) return DASH_OK;  // nothing to launch, as dash_attn_bwd
  if (!table) return DASH_ERR_NULL;
  if (!aligned(table, 4)) return DASH_ERR_SHAPE;
  const int T = dash_attn_tile_size(S, D);
  const int N = (S + T - 1) / T;
  const long long n = dash_schedule_table_tasks(mask, N, Hq / Hkv);
  if (items < 1 || (long long)items > (long long)N * (Hq / Hkv) || n < 0) return DASH_ERR_TABLE;
  if (table_bytes < ((size_t)dash::table_task_words(items) + 2 * (size_t)n) * sizeof(unsigned))
    return DASH_ERR_TABLE;
  DeviceInfo* dev = nullptr;
  st = device_info(&dev);
  if (st != DASH_OK) return st;
  const int full = dev->cus * blocks_per_cu(*dev, D, T, mask);
  if (full <= 0) return DASH_ERR_HIP;
  if (grid < 0 || grid > full) return DASH_ERR_SHAPE;
  const TableArgs tab = {table, items, grid};
  BwdPlan P;
  bool empty = false;
  st = plan_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, S, D, mask, DASH_SCHED_TABLE, workspace,
                workspace_bytes, phases, &P, &empty, &tab);
  if (st != DASH_OK || empty) return st;
  hipStream_t s = (hipStream_t)stream;
  if (phases & 1) {
    st = launch_prepare(P, s);
    if (st != DASH_OK) return st;
  }
  return launch_main_phase(P, D, mask, s);
}

// dash_attn_bwd; `allow_table` = false keeps AUTO among the closed forms
// (no pinned host memory is allocated), for dash_attn_bwd_noalloc.
int bwd_all(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
            void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S, int D, int mask, int schedule,
            void* workspace, size_t workspace_bytes, void* stream, bool allow_table) {
  BwdPlan P;
  bool empty = false;
  int st = plan_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, S, D, mask, schedule, workspace,
                    workspace_bytes, 3, &P, &empty, nullptr, allow_table);
  if (st != DASH_OK || empty) return st;
  hipStream_t s = (hipStream_t)stream;
  st = launch_prepare(P, s);
  if (st != DASH_OK) return st;
  return launch_main_phase(P, D, mask, s);
}

}  // namespace

extern "C" {

int dash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S,
                  int D, int mask, int schedule, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return bwd_all(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, S, D, mask, schedule, workspace,
                 workspace_bytes, stream, true);
}

int dash_attn_bwd_prepare(const void* o, const void* dout, const float* lse, int B, int Hq,
                          int Hkv, int S, int D, int mask, int schedule, void* workspace,
                          size_t workspace_bytes, void* stream) {
  BwdPlan P;
  bool empty = false;
  int st = plan_bwd(nullptr, nullptr, nullptr, o, dout, lse, nullptr, nullptr, nullptr, B, Hq,
                    Hkv, S, D, mask, schedule, workspace, workspace_bytes, 1, &P, &empty);
  if (st != DASH_OK || empty) return st;
  return launch_prepare(P, (hipStream_t)stream);
}

int dash_attn_bwd_run(const void* q, const void* k, const void* v, const void* dout, void* dq,
                      void* dk, void* dv, int B, int Hq, int Hkv, int S, int D, int mask,
                      int schedule, void* workspace, size_t workspace_bytes, void* stream) {
  BwdPlan P;
  bool empty = false;
  int st = plan_bwd(q, k, v, nullptr, dout, nullptr, dq, dk, dv, B, Hq, Hkv, S, D, mask,
                    schedule, workspace, workspace_bytes, 2, &P, &empty);
  if (st != DASH_OK || empty) return st;
  return launch_main_phase(P, D, mask, (hipStream_t)stream);
}

int dash_attn_bwd_table(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int Hq, int Hkv, int S, int D, int mask, const void* table,
                        size_t table_bytes, int items, int grid, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return table_phases(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, S, D, mask, table, table_bytes, items,
                      grid, workspace, workspace_bytes, stream, 3);
}

int dash_attn_bwd_table_run(const void* q, const void* k, const void* v, const void* dout, void* dq,
                            void* dk, void* dv, int B, int Hq, int Hkv, int S, int D, int mask,
                            const void* table, size_t table_bytes, int items, int grid, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return table_phases(q, k, v, nullptr, dout, nullptr, dq, dk, dv, B, Hq, Hkv, S, D, mask, table, table_bytes,
                      items, grid, workspace, workspace_bytes, stream, 2);
}

int dash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          int B, int Hq, int Hkv, int S, int D, int mask, int schedule,
                          void* stream) {
  int st = check_shape(B, Hq, Hkv, S, D, mask, schedule);
  if (st != DASH_OK) return st;
  Layout L;
  st = make_layout(B, Hq, Hkv, S, D, mask, schedule, &L);
  if (st != DASH_OK) return st;
  // the static workspace is fixed in size: larger problems are refused
  // before anything touches the device
  if (L.total > dash::kScratchBytes) return DASH_ERR_WORKSPACE;
  // an empty problem launches nothing and never looks at the workspace
  if (B == 0 || S == 0)
    return bwd_all(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, S, D, mask, schedule, nullptr, 0, stream,
                   false);
  void* ws = nullptr;
  if (dash::scratch_workspace(&ws) != hipSuccess) return DASH_ERR_HIP;
  return bwd_all(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, S, D, mask, schedule, ws, dash::kScratchBytes,
                 stream, false);
}

int dash_attn_bwd_check(const void* workspace, void* stream) {
  if (!workspace) return DASH_ERR_NULL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DASH_ERR_HIP;
  // ctrl[1] error flag, [2] timed-out waits, [3] always zero, [4] not-prepared
  // mark, [5] table-refused mark ([6]: per-head partials written)
  int flag[5] = {0, 0, 0, 0, 0};
  if (hipMemcpy(flag, (const int*)workspace + 1, sizeof(flag), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return DASH_ERR_HIP;
  if (flag[3]) return DASH_ERR_NOT_PREPARED;
  if (flag[4]) return DASH_ERR_TABLE;
  return flag[0] ? DASH_ERR_TIMEOUT : DASH_OK;
}

int dash_attn_bwd_wait_stats(const void* workspace, size_t workspace_bytes, void* stream,
                             long long* waits, long long* polls, double* wait_seconds) {
  if (!workspace) return DASH_ERR_NULL;
  if (workspace_bytes < 256 + (size_t)dash::kWaitSlots * 4 * sizeof(unsigned long long))
    return DASH_ERR_WORKSPACE;
  DeviceInfo* dev = nullptr;
  const int st = device_info(&dev);
  if (st != DASH_OK) return st;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DASH_ERR_HIP;
  std::vector<unsigned long long> v((size_t)dash::kWaitSlots * 4);
  // the wait counters sit right after the 256 bytes of control words
  if (hipMemcpy(v.data(), (const char*)workspace + 256, v.size() * sizeof(v[0]),
                hipMemcpyDeviceToHost) != hipSuccess)
    return DASH_ERR_HIP;
  unsigned long long n = 0, p = 0, t = 0;
  for (int s = 0; s < dash::kWaitSlots; ++s) {
    n += v[4 * s];
    p += v[4 * s + 1];
    t += v[4 * s + 2];
  }
  if (waits) *waits = (long long)n;
  if (polls) *polls = (long long)p;
  if (wait_seconds) *wait_seconds = (double)t / (1000.0 * (double)dev->wall_khz);
  return DASH_OK;
}

int dash_attn_set_watchdog(double seconds) {
  if (!(seconds >= 0.0 && seconds <= 3600.0)) return DASH_ERR_SHAPE;  // also NaN
  g_watchdog_us.store((long long)(seconds * 1e6));
  return DASH_OK;
}

int dash_schedule_num_items(int mask, int schedule, int N) {
  if (N < 1 || (mask != 0 && mask != 1) || schedule < 0 || schedule > 4) return -1;
  if (schedule == DASH_SCHED_SYMMETRIC_SHIFT && (mask != DASH_MASK_CAUSAL || N % 2)) return -1;
  return dash::items_per_group(mask, schedule, N);
}

int dash_schedule_item_len(int mask, int schedule, int N, int G, int item) {
  const int n = dash_schedule_num_items(mask, schedule, N);
  if (n < 0 || G < 1 || item < 0 || item >= n) return -1;
  return dash::item_len(mask, schedule, N, G, item);
}

int dash_schedule_task(int mask, int schedule, int N, int G, int item, int step, int* g, int* i,
                       int* j, int* rank) {
  const int len = dash_schedule_item_len(mask, schedule, N, G, item);
  if (len < 0 || step < 0 || step >= len || !g || !i || !j || !rank) return -1;
  const dash::Task t = dash::task_at(mask, schedule, N, G, item, step);
  *g = t.g;
  *i = t.i;
  *j = t.j;
  *rank = t.rank;
  return 0;
}

}  // extern "C"
