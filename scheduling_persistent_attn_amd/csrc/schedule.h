// Closed-form tile schedules, evaluated identically on the host and in the
// kernels.
//
// A group is one (batch, key/value head); it has N key/value tiles i, N query
// tiles j and G query heads g.  Task (g, i, j) is the work of KV tile i on Q
// tile j of query head g; a causal mask keeps j >= i only.  One *item* is what
// a persistent workgroup takes at a time: the chain of one KV tile over all G
// heads, or for the symmetric shift the pair of KV tiles p and N-1-p.  Keeping
// a KV tile's tasks contiguous on one unit keeps its dK/dV in registers
// (DASH technical summary, section 2.1, constraints).
//
// rank(g, i, j) is the position of KV tile i in the fixed reduction order of
// dQ tile (g, j):
//   NAIVE / DESCENDING_Q : i, ascending KV order (section 1's rigid order;
//                          section 2.2 A only reverses the walk over Q tiles)
//   SHIFT, full          : (j - i) mod N -- chain i reaches Q tile j at step
//                          (j - i) mod N of the cyclic walk i, i+1, ..., i-1
//                          (section 2.2 B), so in lockstep every dQ tile is met
//                          by exactly one chain per step, in this order
//   SHIFT, causal        : j - i (the same walk without the masked tiles)
//   SYMMETRIC_SHIFT      : phase 1 (dense block KV < N/2, Q >= N/2, cyclic):
//                          (j - N/2 - i) mod N/2; phase 2 (the folded
//                          triangles): j - i for Q < N/2, i for KV >= N/2
//                          (section 2.2 B, symmetric shift; the fold geometry
//                          is this library's reading of the two phases).
// Item task lists for G > 1: every step of the single-head list is taken for
// all G heads in turn (step outer, head inner) -- for the symmetric pair part
// by part: phase 1, the KV-p part of phase 2, the KV-(N-1-p) part.  This keeps
// each KV tile's run contiguous and the lockstep free of conflicts with the
// same ranks as one head, and it spaces consecutive contributors to any dQ
// tile a uniform G tasks apart, the most slack against drift between items.
#pragma once

#ifdef __HIPCC__
#define DASH_HD __host__ __device__ inline __attribute__((always_inline))
#else
#define DASH_HD inline
#endif

namespace dash {

enum { MASK_FULL = 0, MASK_CAUSAL = 1 };
// SCHED_TABLE: a schedule written out as a task table (see below).
enum { SCHED_NAIVE = 0, SCHED_DESC = 1, SCHED_SHIFT = 2, SCHED_SYM = 3, SCHED_ATOMIC = 4, SCHED_TABLE = 6 };

struct Task {
  int g, i, j, rank;
  int seg_begin;  // first task of a KV tile's run inside the item
  int seg_end;    // last task of that run
};

// Items built from the symmetric pairs of section 2.2 B: the symmetric shift,
// and the atomic reference on causal masks with an even tile count (its
// result does not depend on the order, so it takes the best-balanced items).
DASH_HD bool paired_items(int mask, int schedule, int N) {
  return schedule == SCHED_SYM || (schedule == SCHED_ATOMIC && mask == MASK_CAUSAL && N % 2 == 0);
}

DASH_HD int items_per_group(int mask, int schedule, int N) {
  return paired_items(mask, schedule, N) ? N / 2 : N;
}

// Tasks of one KV chain per query head.
DASH_HD int chain_len(int mask, int N, int i) { return mask == MASK_CAUSAL ? N - i : N; }

DASH_HD int item_len(int mask, int schedule, int N, int G, int item) {
  if (paired_items(mask, schedule, N)) return G * (N + 1);
  return G * chain_len(mask, N, item);
}

// Number of key/value tiles reducing into any dQ tile j.
DASH_HD int contributors(int mask, int N, int j) { return mask == MASK_CAUSAL ? j + 1 : N; }

DASH_HD Task task_at(int mask, int schedule, int N, int G, int item, int step) {
  Task t;
  if (paired_items(mask, schedule, N)) {
    const int h = N / 2, p = item;
    const int len_a = G * (N - p);  // phase 1 + KV-p part of phase 2
    if (step < len_a) {
      t.i = p;
      t.seg_begin = step == 0;
      t.seg_end = step == len_a - 1;
      if (step < G * h) {
        const int s = step / G;
        t.g = step - s * G;
        t.j = h + (p + s) % h;
        t.rank = s;
      } else {
        const int k = step - G * h;
        const int s = k / G;
        t.g = k - s * G;
        t.j = p + s;
        t.rank = s;
      }
    } else {
      const int k = step - len_a, l2 = p + 1;
      t.i = N - 1 - p;
      t.seg_begin = k == 0;
      t.seg_end = k == G * l2 - 1;
      const int s = k / G;
      t.g = k - s * G;
      t.j = N - 1 - s;
      t.rank = t.i;
    }
    // the atomic reference keeps the ascending key/value order of ranks
    if (schedule == SCHED_ATOMIC) t.rank = t.i;
    return t;
  }
  const int i = item;
  const int L = chain_len(mask, N, i);
  t.i = i;
  const int s = step / G;
  t.g = step - s * G;
  t.seg_begin = step == 0;
  t.seg_end = step == G * L - 1;
  const int first = mask == MASK_CAUSAL ? i : 0;
  switch (schedule) {
    case SCHED_DESC:
      t.j = N - 1 - s;
      t.rank = i;
      break;
    case SCHED_SHIFT:
      t.j = mask == MASK_CAUSAL ? i + s : (i + s) % N;
      t.rank = s;
      break;
    default:  // NAIVE, ATOMIC
      t.j = first + s;
      t.rank = i;
      break;
  }
  return t;
}

// Packed device form of a task table (one group's items; every group runs
// the same table).  Words: a header of kTableHeaderWords -- magic, N, G,
// mask (| kTableSplit for the per-head form), passes per task, items, widest
// dispatch block, tasks -- then the item offsets (items + 1 words, padded to
// an even count), then two words per task: i | j << 16 and
// g | rank << 16 | run start << 30 | run end << 31, where a run is a
// key/value tile's unbroken stretch of tasks in its item (in the per-head
// form, one head's: its dK/dV leave the unit as that head's fp32 partial).
// The kernels compare the header with their launch and refuse a table made
// for another shape or kernel, or a launch with fewer workgroups than the
// table's widest dispatch block.
constexpr int kTableHeaderWords = 8;
constexpr unsigned kTableMagic = 0x54485344u;  // "DSHT"
constexpr unsigned kTableSplit = 0x100u;       // header word 3: per-head runs

// Word index of the first task, after the header and the item offsets.
DASH_HD int table_task_words(int items) { return kTableHeaderWords + ((items + 2) & ~1); }

DASH_HD Task table_task(unsigned w0, unsigned w1) {
  Task t;
  t.i = (int)(w0 & 0xffffu);
  t.j = (int)(w0 >> 16);
  t.g = (int)(w1 & 0xffffu);
  t.rank = (int)((w1 >> 16) & 0x3fffu);
  t.seg_begin = (int)((w1 >> 30) & 1u);
  t.seg_end = (int)(w1 >> 31);
  return t;
}

}  // namespace dash
