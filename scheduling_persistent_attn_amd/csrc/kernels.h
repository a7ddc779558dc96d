// Kernel parameter blocks and launch entry points shared by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace dash {

// Wave slots of the turn-wait counters: the workspace region right after the
// 64 control words, 4 uint64 per slot.
constexpr int kWaitSlots = 4096;

struct PreParams {
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;      // [B*Hq][NT]: -rowsum(dO * O), 0 past S
  float* lse2;       // [B*Hq][NT]: -lse / scale, -inf past S
  int* counters;     // n_counters ints, zeroed
  int* ctrl;         // 64 ints, zeroed
  unsigned long long* waits;  // kWaitSlots x 4, zeroed
  float* dqacc;      // zeroed when zero_dqacc (atomic schedule)
  long long n_counters;
  long long n_dqacc;
  int zero_dqacc;
  float inv_scale;   // 1 / softmax scale
  int B, Hq, S, D, NT;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const float* delta;  // -Dl per padded query row
  const float* lse2;   // -lse / scale per padded query row
  float* dqacc;
  int* counters;
  int* ctrl;
  int B, Hq, Hkv, S, N, G;
  int mask, schedule;
  int total_items, items_per_group;
  // Query heads of a group split over `parts` items per base item (chain or
  // symmetric pair): item `local` of a group is part local / base_items (its
  // heads part*Gp .. part*Gp + Gp - 1) of base item local % base_items.  With
  // parts > 1 each item writes fp32 partial dK/dV to dkv_part, summed by
  // bwd_dkv_finalize in ascending part order.
  int parts, Gp, base_items;
  float* dkv_part;     // [2][B][Hkv][parts][NT][D] fp32 (dK then dV); parts > 1
  int NT;              // N * T: rows of the padded sequence
  // Table schedules: the packed task table (layout in schedule.h; caller's
  // device memory) and its tasks per group.  NULL / 0 otherwise.
  const unsigned* table;
  int table_tasks;
  float scale, scale_log2e;
  long long spin_ticks;
  // Task trace of the debug build (compiled with DASH_TASK_TRACE; NULL
  // otherwise): record item * trace_len + step (for a table schedule, the
  // task's index group * table_tasks + its table index), 8 uint64 each -- [0] item |
  // step << 32, [1] g | i << 16 | j << 32 | rank << 48, [2] workgroup, [3]
  // and [4] the 100 MHz wall clock when the task starts and ends.
  unsigned long long* trace;
  int trace_len;
};

#ifdef DASH_TASK_TRACE
// Start of a task's trace record (thread 0 of the workgroup; vector stores).
__device__ __forceinline__ unsigned long long* trace_begin(const BwdParams& p, long long rec, int item, int step,
                                                          int g, int i, int j, int rank) {
  unsigned long long* r = p.trace + rec * 8;
  if (threadIdx.x == 0) {
    r[0] = (unsigned)item | ((unsigned long long)(unsigned)step << 32);
    r[1] = (unsigned long long)(unsigned)g | ((unsigned long long)(unsigned)i << 16) |
           ((unsigned long long)(unsigned)j << 32) | ((unsigned long long)(unsigned)rank << 48);
    r[2] = blockIdx.x;
    r[3] = wall_clock64();
  }
  return r;
}
__device__ __forceinline__ void trace_end(unsigned long long* r) {
  if (threadIdx.x == 0) r[4] = wall_clock64();
}
#endif

struct DkvFinParams {
  const float* dkv_part;  // as in BwdParams
  void* dk;
  void* dv;
  const int* ctrl;        // the error flag ctrl[1] up: write nothing
  int B, Hkv, S, NT, D, parts;
  int need_mark;          // write only if control word 6 is set (a table run
                          // marks it when its per-head partials are written)
  float scale;            // dK = scale * sum over the parts
};

struct FinParams {
  const float* dqacc;
  const int* ctrl;   // the error flag ctrl[1] up: write nothing
  void* dq;
  int B, Hq, S, N;
  float scale;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, S, G;
  float scale_log2e;
};

// Bytes of the static device workspace behind dash_attn_bwd_noalloc.
constexpr size_t kScratchBytes = (size_t)64 << 20;

// Device address of this GPU's static workspace (looked up once per device,
// on the current device).
hipError_t scratch_workspace(void** out);

// Persistent workgroups per compute unit for the backward kernel of (D, T,
// causal); 0 if not instantiated.
int bwd_blocks_per_cu(int D, int T, bool causal);
int bwd_block_threads(int T);

// The 256-key tile kernel (head dim 128; bwd_wide.hip).
int bwd_wide_blocks_per_cu(bool causal);
hipError_t launch_bwd_wide(bool causal, const BwdParams& p, int grid, hipStream_t s);
hipError_t launch_finalize_wide(const FinParams& p, hipStream_t s);

// The 256-key tile kernel for head dim 64 (bwd_wide64.hip).
int bwd_wide64_blocks_per_cu(bool causal);
hipError_t launch_bwd_wide64(bool causal, const BwdParams& p, int grid, hipStream_t s);
hipError_t launch_finalize_wide64(const FinParams& p, hipStream_t s);

hipError_t launch_dkv_finalize(const DkvFinParams& p, hipStream_t s);

hipError_t launch_preprocess(const PreParams& p, hipStream_t s);
hipError_t launch_bwd_main(int D, int T, bool causal, const BwdParams& p, int grid,
                           hipStream_t s);
hipError_t launch_finalize_atomic(int D, int T, const FinParams& p, hipStream_t s);
hipError_t launch_fwd(int D, bool causal, const FwdParams& p, hipStream_t s);

}  // namespace dash
