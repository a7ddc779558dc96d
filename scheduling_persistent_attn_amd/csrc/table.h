// Task tables: a schedule written out task by task, so that any order the
// search below finds (or a caller writes) runs on the device.  The DASH
// technical summary frames scheduling as minimising the critical path of the
// backward DAG (section 2.1) and leaves the choice per shape and hardware to
// the practitioner (section 2); the closed forms of schedule.h are points of
// the family searched here.
#pragma once

#include <stdint.h>

#include <vector>

#include "../../include/dash_attn.h"

#include "schedule.h"

namespace dash {

struct TableTask {
  int g, i, j, rank;
};

// One group's items: item k is tasks[offs[k] .. offs[k+1]).  A run is an
// unbroken stretch of one key/value tile's tasks in an item (the unit keeps
// that tile's dK/dV in registers): in the whole-tile form one run per
// key/value tile holds all its heads; in the per-head form (split) one run
// per (query head, key/value tile), whose dK/dV leave the unit as that head's
// fp32 partial.
struct GroupTable {
  std::vector<int> offs;
  std::vector<TableTask> tasks;
  bool split = false;
};

// Whether task t + 1 continues task t's run.
inline bool same_run(const GroupTable& tb, size_t t) {
  return tb.tasks[t + 1].i == tb.tasks[t].i && (!tb.split || tb.tasks[t + 1].g == tb.tasks[t].g);
}

// Tiles of one query head (full: N*N, causal: N(N+1)/2).
long long table_tiles(int mask, int N);

// Structural checks of a table (every tile of every head exactly once, the
// ranks of each dQ tile a permutation, and either each key/value tile's tasks
// one contiguous run inside one item -- the whole-tile form, preferred when
// both hold -- or each (head, key/value tile)'s tasks one such run -- the
// per-head form); on success fills *out (with its form) and, if `packed` is
// given, the device form: two words per task, i | j << 16 and
// g | rank << 16 | run start << 30 | run end << 31.
int table_validate(int mask, int N, int G, int items, const int* offs, const int* tasks, GroupTable* out,
                   std::vector<uint32_t>* packed);

// Whether the kernels' ordered hand-offs can always finish on P persistent
// workgroups with `passes` passes per task (see table.cpp).  *blocks gets the
// number of dispatch blocks, *widest the largest.  DASH_OK or DASH_ERR_TABLE.
int table_protocol(int mask, int N, const GroupTable& t, int passes, int P, int* blocks, int* widest);

// Critical path of a table schedule on `groups` copies of the group, P
// workers (the same model and report as dash_sim_run).
int sim_table(int mask, int N, int G, int groups, int P, int dispatch, double c_full, double c_diag, double r,
              const GroupTable& t, dash_sim_result* out);

// The closed-form schedules of schedule.h as tables.
GroupTable closed_form_table(int mask, int schedule, int N, int G);

// Passes per task of the kernel for tiles of T keys at head dim D.
int passes_per_task(int T, int D);

// The searched family (see table.cpp).  For DASH_FAMILY_PACKED `block` is
// the number of bins.
bool family_applies(int mask, int N, int kind);
GroupTable family_table(int mask, int N, int G, int kind, int order, int block);
std::vector<int> family_blocks(int units, int P);

// Bins of the packed family for `groups` groups on P workgroups: the
// workgroups one group gets, at most the G * N chains.
int packed_bins(int N, int G, int groups, int P);

}  // namespace dash
