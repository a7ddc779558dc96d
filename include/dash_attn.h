/*
 * dash_attn.h -- deterministic attention backward for AMD MI355X (gfx950).
 *
 * C ABI of libdash_attn.so.  Plain pointers and sizes only.
 *
 * The method: the softmax-attention backward computed tile by tile with the
 * dK/dV of one key/value tile kept in registers while the unit walks that
 * tile's query tiles (a "chain"), and with dQ accumulated across key/value
 * tiles in a fixed order so that results are bitwise reproducible.  Sources:
 * "DASH: Deterministic Attention Scheduling for High-throughput Reproducible
 * LLM Training", explained on gist.science (technical summary in Spanish and
 * Chinese, lay explanation in French); section numbers below refer to the
 * technical summary.
 *
 * Tensor layouts (all device pointers, bf16 = IEEE bfloat16, row-major,
 * contiguous, 16-byte aligned):
 *   q, o, dout, dq : [B, S, Hq,  D] bf16
 *   k, v, dk, dv   : [B, S, Hkv, D] bf16
 *   lse            : [B, Hq, S]     fp32, natural-log log-sum-exp of the
 *                                    scaled, masked scores of each query row
 * Query head h reads key/value head h / (Hq / Hkv).  The softmax scale is
 * 1/sqrt(D).  Causal masking hides key positions after the query position
 * (equal query and key lengths).  Supported: D in {64, 128}; any S >= 0
 * (the last tile may be partial); Hq a positive multiple of Hkv.
 *
 * Ownership: the caller owns every buffer, including the workspace (size from
 * dash_attn_bwd_workspace_size).  The library allocates no device memory; it
 * caches the device's compute-unit count and the kernels' occupancy, and
 * DASH_SCHED_AUTO's choice per device and shape (with, where that choice is
 * the searched task table, the table's device form in pinned host memory,
 * allocated on the shape's first AUTO call and held until the process ends;
 * dash_attn_bwd_noalloc never makes that choice).  The caches are guarded by
 * locks.  Calls are asynchronous on the given HIP stream (NULL = default
 * stream).
 *
 * Errors: every argument is checked on the host before anything is enqueued;
 * a non-zero status means nothing was launched.  A failed kernel launch
 * returns DASH_ERR_HIP.  A device-side watchdog turns a stalled ordered
 * reduction into an error flag in the workspace, reported by
 * dash_attn_bwd_check as DASH_ERR_TIMEOUT (the outputs are then undefined).
 */
#ifndef DASH_ATTN_H
#define DASH_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dash_mask { DASH_MASK_FULL = 0, DASH_MASK_CAUSAL = 1 };

/* Tile schedules of the backward pass (technical summary, section 2.2).
 *  NAIVE            each key/value chain walks its query tiles upward; every
 *                   dQ tile is reduced in ascending key/value order (the rigid
 *                   order of section 1 that the method improves on).
 *  DESCENDING_Q     chains walk their query tiles from the last to the first
 *                   (section 2.2 A); same reduction order as NAIVE.
 *  SHIFT            chain i visits query tiles i, i+1, ..., N-1, 0, ..., i-1
 *                   (section 2.2 B, full masks); every dQ tile is reduced in
 *                   the order the chains reach it in lockstep.  With a causal
 *                   mask the masked tiles of the cycle are skipped.
 *  SYMMETRIC_SHIFT  causal masks with an even tile count: key/value tiles p
 *                   and N-1-p share one unit; a dense phase over
 *                   {KV < N/2} x {Q >= N/2}, then the two folded triangles
 *                   (section 2.2 B, symmetric shift).
 *  ATOMIC           NOT deterministic: dQ reduced with unordered fp32 atomic
 *                   adds (the non-deterministic counterpart of section 1);
 *                   kept only as the speed reference.  Its items are the
 *                   symmetric pairs on causal masks with an even tile count
 *                   (the best-balanced items; its result does not depend on
 *                   the order), one chain per KV tile otherwise; ranks are
 *                   reported in ascending KV order.
 *  AUTO             one of the four deterministic schedules, or the
 *                   library's searched task table, chosen per shape and
 *                   device by the schedule simulator below (see
 *                   dash_attn_bwd_auto_schedule); deterministic like the
 *                   schedule it resolves to.
 *  TABLE            a deterministic schedule written out task by task (a
 *                   searched one, see dash_schedule_search); run only by
 *                   dash_attn_bwd_table.  dash_attn_bwd_workspace_size and
 *                   dash_attn_bwd_prepare accept it.
 */
enum dash_schedule {
  DASH_SCHED_NAIVE = 0,
  DASH_SCHED_DESCENDING_Q = 1,
  DASH_SCHED_SHIFT = 2,
  DASH_SCHED_SYMMETRIC_SHIFT = 3,
  DASH_SCHED_ATOMIC = 4,
  DASH_SCHED_AUTO = 5,
  DASH_SCHED_TABLE = 6
};

enum dash_status {
  DASH_OK = 0,
  DASH_ERR_NULL = 1,          /* a required pointer is NULL                 */
  DASH_ERR_SHAPE = 2,         /* negative size, Hq % Hkv != 0, misaligned    */
  DASH_ERR_UNSUPPORTED = 3,   /* head dim, or a schedule that needs a whole
                                 group of chains resident at once on more
                                 units than the device runs concurrently    */
  DASH_ERR_SCHEDULE_MASK = 4, /* unknown mask/schedule, or SYMMETRIC_SHIFT
                                 with a full mask or an odd tile count       */
  DASH_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than required     */
  DASH_ERR_HIP = 6,           /* a HIP runtime call or launch failed         */
  DASH_ERR_TIMEOUT = 7,       /* the device watchdog fired during a backward */
  DASH_ERR_NOT_PREPARED = 8,  /* dash_attn_bwd_run found a workspace that
                                 dash_attn_bwd_prepare had not reset since
                                 the previous run; nothing was computed      */
  DASH_ERR_TABLE = 9          /* a task table that does not cover every tile
                                 of every head once, whose ranks are not a
                                 permutation per dQ tile, that splits a
                                 key/value tile's tasks, or whose hand-offs
                                 could wait forever (see
                                 dash_schedule_table_check); from
                                 dash_attn_bwd_check: the kernel refused the
                                 table, nothing was computed                 */
};

/* Query-tile and key/value-tile edge T used for a problem (both sides use the
 * same T): for D == 64, 64 when S <= 512, else 256; for D == 128, 128 when
 * S <= 512, else 256 (a unit then holds the dK/dV of 256 keys, which halves
 * the bytes moved per FLOP against 128-key tiles).  Returns 0 if D is
 * unsupported. */
int dash_attn_tile_size(int S, int D);

/* Number of parts the query heads of each (batch, key/value head) group are
 * split into, a function of the arguments alone (0 if invalid).  Normally 1:
 * one item serves a key/value tile (or symmetric pair) for all G = Hq/Hkv
 * query heads, so dK/dV are summed in registers.  With 256-key tiles a launch
 * can have fewer items than an MI355X has compute units (256); then the heads
 * are split into `parts` runs of G/parts consecutive heads -- the smallest
 * divisor of G that gives at least 256 items, else G -- and every item
 * exists once per part, serving only that part's heads.  Items are dispatched
 * group by group, part by part, so the items of one part run together (the
 * shift family needs that).  Each part writes its fp32 dK/dV to the workspace
 * and a final pass sums the parts in ascending order.  For AUTO, the largest
 * over the schedules it can resolve to. */
int dash_attn_bwd_head_parts(int B, int Hq, int Hkv, int S, int D, int mask, int schedule);

/* Bytes of workspace dash_attn_bwd needs for these arguments, or 0 if the
 * arguments are invalid.  Layout (offsets rounded up to 256 bytes):
 *   ctrl      64 x int32   [0] work-dispatch counter, [1] error flag
 *                          (watchdog, not prepared or table refused), [2]
 *                          number of waits that timed out, [3] always
 *                          zero, [4] set when a run found the workspace not
 *                          prepared, [5] set when the kernel refused a task
 *                          table (dash_attn_bwd_table), [6] set when a
 *                          per-head table wrote its fp32 dK/dV partials,
 *                          [8..15]
 *                          four uint64: shader-clock and 100 MHz-clock
 *                          stamps of workgroup 0 at the persistent kernel's
 *                          start and exit (their ratio is the clock it ran at)
 *   waits     4096 x 4 uint64: per wave of the persistent grid (slot =
 *             workgroup * waves per workgroup + wave), the turn waits that
 *             found the turn not yet taken: [0] count, [1] polls, [2]
 *             wall-clock ticks spent (dash_attn_bwd_wait_stats sums them)
 *   counters  B*Hq*N*W int32: the turn counter of every (batch, query head,
 *             dQ tile, slice) -- a slice is the block of the tile one wave
 *             reduces per pass; after a deterministic backward each holds the
 *             number of key/value tiles that reduced into that dQ tile
 *             (N = ceil(S/T))
 *   delta     B*Hq*N*T fp32: -rowsum(dout * o), zero past S
 *   lse2      B*Hq*N*T fp32: -lse / scale, -inf past S
 *   dqacc     B*Hq*N*T*D fp32: dQ partial sums in the kernels' lane order
 *   dkvp      only when the heads are split (dash_attn_bwd_head_parts > 1):
 *             2*B*Hkv*parts*N*T*D fp32, each part's dK then dV sums
 * (W = T*D/1024 for tiles of 64 and 128: one counter per 32 x 32 slice; W =
 * T*D/512 for 256: one per 32 x 16 slice.)
 */
size_t dash_attn_bwd_workspace_size(int B, int Hq, int Hkv, int S, int D,
                                    int mask, int schedule);

/* Attention forward (support for the backward): o = softmax(scale*q k^T +
 * mask) v in bf16 (round to nearest even) and lse in fp32.  Overwrites o and
 * lse.  Not part of the deterministic-reduction contract, but itself
 * deterministic (no cross-workgroup reduction).  Layouts, alignment and the
 * shape errors are those of dash_attn_bwd; DASH_ERR_UNSUPPORTED also when
 * B*S*Hq*D >= 2^31 (the kernel forms 32-bit offsets) or B > 65535. */
int dash_attn_fwd(const void* q, const void* k, const void* v, void* o,
                  float* lse, int B, int Hq, int Hkv, int S, int D, int mask,
                  void* stream);

/* Attention backward: overwrites dq, dk, dv (bf16, round to nearest even)
 * with the gradients of sum(dout * o) with respect to q, k, v, given the
 * forward's o and lse.  Arithmetic: bf16 operands, fp32 accumulation; P and
 * dS are rounded to bf16 before their products.
 *
 * Determinism contract (schedules 0-3): for fixed inputs, shape, mask,
 * schedule and library binary, dq/dk/dv are bitwise identical across calls,
 * streams and timing.  Different schedules may differ in the last bits.
 * dK/dV of a key/value tile are summed over its query heads inside one unit,
 * in the unit's fixed task order (each query tile of the walk taken for all
 * heads in turn); when the heads are split into parts (see
 * dash_attn_bwd_head_parts) each part is summed that way and the parts are
 * then added in ascending order.  The dQ tile j of query head h is reduced in the order given
 * by the schedule (see enum dash_schedule) using per-tile turn counters in
 * the workspace.
 *
 * The workspace must not be shared by concurrently running calls.  Backward
 * calls that overlap in time on one device (different streams with no
 * ordering between them) share its compute units: the shift family needs a
 * whole group of items resident at once, so two such calls near the residency
 * limit can each hold units the other's items wait for.  Nothing hangs (every
 * wait is bounded by the watchdog), but the calls then fail with
 * DASH_ERR_TIMEOUT; order such calls with a stream or events. */
int dash_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk,
                  void* dv, int B, int Hq, int Hkv, int S, int D, int mask,
                  int schedule, void* workspace, size_t workspace_bytes,
                  void* stream);

/* The two phases of dash_attn_bwd, for callers that want to schedule or time
 * them separately (same arguments and checks; pointers a phase does not read
 * may be NULL).
 *
 * dash_attn_bwd_prepare: the per-row values of the standard attention
 * backward -- -rowsum(dout * o) and -lse/scale into the workspace -- and the
 * reset of the work-dispatch counter, the watchdog flag and every turn
 * counter (and, for ATOMIC, the dQ accumulator).
 *
 * dash_attn_bwd_run: the persistent backward over the schedule's items (and,
 * for ATOMIC, the pass that converts the fp32 accumulator to bf16 dq).  It
 * requires that dash_attn_bwd_prepare ran on this workspace, with the same
 * shape, mask and schedule, after the previous run.  A run on a workspace
 * that was not prepared again after an earlier run finds the dispatch
 * counter already used: it computes nothing, leaves dq/dk/dv untouched, and
 * dash_attn_bwd_check then returns DASH_ERR_NOT_PREPARED.  (A prepare with a
 * different shape, mask or schedule is not detected; the results are then
 * undefined.) */
int dash_attn_bwd_prepare(const void* o, const void* dout, const float* lse, int B,
                          int Hq, int Hkv, int S, int D, int mask, int schedule,
                          void* workspace, size_t workspace_bytes, void* stream);

int dash_attn_bwd_run(const void* q, const void* k, const void* v,
                      const void* dout, void* dq, void* dk, void* dv, int B,
                      int Hq, int Hkv, int S, int D, int mask, int schedule,
                      void* workspace, size_t workspace_bytes, void* stream);

/* dash_attn_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device array
 * of the library, 64 MiB on each GPU the library runs on, held until the
 * process ends; this call allocates nothing, and it clears what must start at
 * zero with kernels (no memset nodes).  Same arguments (less the workspace),
 * results, determinism contract and errors as dash_attn_bwd, plus
 * DASH_ERR_WORKSPACE, before anything is enqueued, when the problem's
 * workspace (dash_attn_bwd_workspace_size) exceeds 64 MiB.  Here AUTO chooses
 * among the four closed forms only (the searched table would need pinned
 * host memory), so it may resolve differently from dash_attn_bwd's AUTO.  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one device race
 * and give undefined results; order them with a stream or events.  The
 * watchdog flag lands in the static array, where dash_attn_bwd_check cannot
 * read it; callers that need it use dash_attn_bwd with a workspace of their
 * own. */
int dash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          int B, int Hq, int Hkv, int S, int D, int mask, int schedule,
                          void* stream);

/* Waits for the stream, then reports DASH_ERR_NOT_PREPARED if the last
 * backward run on this workspace found it not prepared, DASH_ERR_TABLE if the
 * kernel refused its task table, DASH_ERR_TIMEOUT if its watchdog fired,
 * DASH_ERR_HIP on a runtime error, else DASH_OK.  Reads 20 bytes of the
 * workspace. */
int dash_attn_bwd_check(const void* workspace, void* stream);

/* Sums the turn-wait counters the last backward on this workspace left in it
 * (after waiting for the stream): *waits = turn waits that found the turn not
 * yet taken when first checked, *polls = re-polls of their counters, and
 * *wait_seconds = wall-clock time those waits took, summed over the waves
 * that made them.  These are the schedule's bubbles: time a wave could not
 * proceed because an earlier contribution to a dQ tile was not yet added.
 * The atomic reference makes no waits.  Any output pointer may be NULL to
 * skip that figure.  Returns DASH_ERR_NULL without a workspace,
 * DASH_ERR_WORKSPACE if workspace_bytes does not cover the control words and
 * the wait counters (256 + 4096 * 32 bytes), DASH_ERR_HIP on a runtime
 * error. */
int dash_attn_bwd_wait_stats(const void* workspace, size_t workspace_bytes, void* stream,
                             long long* waits, long long* polls, double* wait_seconds);

/* Sets the device watchdog of the ordered reductions for the backward calls
 * planned after it, process-wide: a wave that has waited `seconds` of wall
 * clock for its turn gives up and raises the workspace's error flag; every
 * later wait of that launch then gives up within 64 polls, so the launch
 * drains and dash_attn_bwd_check reports DASH_ERR_TIMEOUT.  The default is
 * 2 s.  0 makes any wait longer than 64 polls time out (a caller can force
 * the error path this way).  Returns DASH_ERR_SHAPE, leaving the setting
 * unchanged, for a negative or non-finite value or one above 3600 s. */
int dash_attn_set_watchdog(double seconds);

/* The deterministic schedule that DASH_SCHED_AUTO resolves to for these
 * arguments on the current device (DASH_SCHED_TABLE for the searched table),
 * or minus a dash_status.  The closed forms are simulated over the device's
 * persistent grid (P = the workgroups dash_attn_bwd launches, dynamic
 * dispatch), B*Hkv groups of Hq/Hkv query heads on the tile count of (S, D),
 * each with its own split of the query heads (a split group simulates as
 * `parts` groups of G/parts heads), with weights c_full = c_diag = 1 (the
 * kernel computes a causal diagonal tile in full) and r = 0.1 (the exposed
 * part of a hand-off, relative to one task); SHIFT and SYMMETRIC_SHIFT are
 * candidates only when one group of items fits in the grid.  The table
 * dash_schedule_search finds with the same grid and weights is a candidate
 * too where it needs no more workspace than the closed forms (64- or
 * 128-key tiles, G = 1, or closed forms that already split the heads into
 * G parts) and the problem simulates at most 2^18 tasks (B*Hkv groups times
 * the tasks of one); it wins only with a strictly shorter critical path.
 * The result is cached per device and shape, so a given shape on a given
 * device always runs the same schedule: AUTO keeps the determinism
 * contract.  When the table is chosen, its device form is kept in pinned
 * host memory (held until the process ends) and every prepare phase copies
 * it into the workspace, on the call's stream; the first call for a shape
 * runs the search on the host (up to about two seconds). */
int dash_attn_bwd_auto_schedule(int B, int Hq, int Hkv, int S, int D, int mask);

/* The same choice on the host alone, for a device whose persistent grid is
 * `grid` workgroups (dash_attn_bwd_grid_size on that device): no device is
 * touched and nothing is cached.  Returns the schedule or minus a
 * dash_status (DASH_ERR_SHAPE for grid < 1 with a non-empty shape). */
int dash_attn_bwd_auto_schedule_on(int B, int Hq, int Hkv, int S, int D, int mask, int grid);

/* Static description of a status code. */
const char* dash_status_string(int status);

/* Number of persistent workgroups the backward launches for these arguments
 * (compute units x resident workgroups per unit), or 0 if invalid / no
 * device.  Queries the current device. */
int dash_attn_bwd_grid_size(int S, int D, int mask);

/* ---------------------------------------------------------------------------
 * Schedule description (host only; the kernels evaluate the same closed forms
 * on the device).  One item is the unit of work a persistent workgroup takes:
 * a key/value chain (NAIVE, DESCENDING_Q, SHIFT, ATOMIC) or a symmetric pair
 * (SYMMETRIC_SHIFT), covering all G query heads of one key/value head.
 */

/* Items per (batch, key/value head) group, or -1 if invalid. */
int dash_schedule_num_items(int mask, int schedule, int N);

/* Tasks in item `item` of a group with G query heads per key/value head, or
 * -1 if invalid. */
int dash_schedule_item_len(int mask, int schedule, int N, int G, int item);

/* Task `step` of item `item`: writes query head g (0..G-1), key/value tile i,
 * query tile j and the rank of that reduction in dQ tile (g, j).  Returns 0,
 * or -1 if out of range. */
int dash_schedule_task(int mask, int schedule, int N, int G, int item,
                       int step, int* g, int* i, int* j, int* rank);

/* ---------------------------------------------------------------------------
 * Schedule simulator (CPU).  Builds the backward DAG of the technical
 * summary's section 2.1 for `groups` independent (batch, key/value head)
 * groups of N x N tiles with G query heads each, placed on P workers, and
 * reports its critical path and the depth condition of Lemma 1 (section 2.2
 * B) on every added accumulation-order edge.
 *
 * Events per task: S, E (compute, weight c, or c_diag on a causal diagonal
 * tile), R, F (reduction, weight r); zero-weight edges E->R, between
 * consecutive tasks of an item, between consecutive items of a worker, and
 * the order edges F(rank q) -> R(rank q+1) of every dQ tile.  depth = longest
 * path from a source.  dispatch 0: item k runs on worker k mod P; 1: the next
 * item goes to the first idle worker (lower index on ties), as on the GPU.
 */
typedef struct {
  double makespan;      /* critical path of the full DAG (+inf on deadlock) */
  double base_makespan; /* critical path without the order edges            */
  double total_work;    /* sum of all compute and reduction weights         */
  double efficiency;    /* total_work / (min(P, items) * makespan)          */
  double max_deficit;   /* largest depth(u) - depth(v) over order edges     */
  long long order_edges;
  long long violations; /* order edges with depth(u) > depth(v)             */
  int deadlock;         /* 1 if the order edges close a cycle or the replay
                           stalls                                           */
} dash_sim_result;

int dash_sim_run(int mask, int schedule, int N, int G, int groups, int P,
                 int dispatch, double c_full, double c_diag, double r,
                 dash_sim_result* out);

/* Schedule selection by critical path (NEXT step of the pages' section 2:
 * pick the strategy per shape and hardware).  Simulates every deterministic
 * schedule that applies to the mask and N (SYMMETRIC_SHIFT only for causal
 * masks and even N), skips those that deadlock on P workers, and writes the
 * one with the shortest critical path to *schedule (ties go to the earlier of
 * SYMMETRIC_SHIFT, SHIFT, DESCENDING_Q, NAIVE) and its report to *out (may be
 * NULL).  Returns DASH_ERR_UNSUPPORTED when every candidate deadlocks, and the
 * argument errors of dash_sim_run. */
int dash_sim_select(int mask, int N, int G, int groups, int P, int dispatch,
                    double c_full, double c_diag, double r, int* schedule,
                    dash_sim_result* out);

/* ---------------------------------------------------------------------------
 * Task tables: a schedule written out task by task (host arrays), searched,
 * checked, packed for the device and run.  The pages frame scheduling as
 * minimising the backward DAG's critical path and leave the choice per shape
 * and hardware open (technical summary, sections 2 and 2.1); the closed forms
 * above are members of the family searched here.
 *
 * A table describes one (batch, key/value head) group; every group runs it.
 *   items          number of items (1..N, 1..G*N in the per-head form below):
 *                  what a workgroup takes at a time
 *   item_offsets   items + 1 ints: item k is tasks item_offsets[k] ..
 *                  item_offsets[k+1] - 1, item_offsets[0] = 0, strictly
 *                  increasing, item_offsets[items] = number of tasks
 *   tasks          4 ints per task: query head g (0..G-1), key/value tile i,
 *                  query tile j, rank (position of this contribution in the
 *                  reduction order of dQ tile (g, j), 0..n_j - 1 where n_j =
 *                  N for a full mask and j + 1 for a causal one)
 * Valid when every unmasked (g, i, j) appears exactly once, the ranks of each
 * dQ tile are a permutation, and all tasks of a key/value tile (every head
 * and query tile) form one unbroken run inside one item (the unit keeps its
 * dK/dV in registers, section 2.1) -- or, in the per-head form, all tasks of
 * each (head, key/value tile) do: then each run's dK/dV leave the unit as
 * that head's fp32 partial and a fixed-order pass adds the G partials of each
 * key row (256-key tiles only; the workspace of DASH_SCHED_TABLE covers them).
 * The whole-tile form is taken when both hold.  Tasks run in item order;
 * dispatch gives items to workgroups in order, group by group.
 *
 * Deadlock freedom on P workgroups (dash_schedule_table_check): the waits-for
 * graph of the kernels' pipelined hand-offs -- within a run the turn of pass
 * n is taken after pass n+1 and the slice published in pass n+3 (passes per
 * task: 8 for 256-key tiles at D = 128, 4 for 256-key tiles at D = 64 and
 * for 128-key tiles, 2 for 64-key tiles) --
 * has no cycle, and the items split into consecutive dispatch blocks of at
 * most P items where no item waits on a later block.
 */

/* Family kinds of dash_schedule_search (family[0]). */
enum dash_family {
  DASH_FAMILY_SYMMETRIC = 0,  /* symmetric pairs (causal, even N)            */
  DASH_FAMILY_SHIFT = 1,      /* cyclic walk from the diagonal (causal: the
                                 diagonal upward)                            */
  DASH_FAMILY_DESCENDING = 2, /* query tiles from the last down              */
  DASH_FAMILY_ASCENDING = 3,  /* query tiles from the first up (full masks)  */
  DASH_FAMILY_PACKED = 4      /* (head, key/value tile) chains packed longest
                                 first into one item per workgroup; reduced
                                 in the order of their no-wait start        */
};

/* Tasks in one group's table: G * N * N (full) or G * N(N+1)/2 (causal);
 * -1 if invalid. */
long long dash_schedule_table_tasks(int mask, int N, int G);

/* A closed-form deterministic schedule (NAIVE .. SYMMETRIC_SHIFT) written as
 * a table; item_offsets needs N + 1 ints, tasks 4 ints per task. */
int dash_schedule_table_closed_form(int mask, int schedule, int N, int G, int* items,
                                    int* item_offsets, int* tasks);

/* One member of the searched family (below) as a table: kind, order (0
 * ascending, 1 descending; the packed kind has order 0 only) and block
 * (dispatch block size in units, or the packed kind's bins).  item_offsets
 * needs G * N + 1 ints, tasks 4 ints per task.  DASH_ERR_SCHEDULE_MASK if the
 * kind does not apply to the mask and N. */
int dash_schedule_table_family(int mask, int N, int G, int kind, int order, int block, int* items,
                               int* item_offsets, int* tasks);

/* DASH_OK if the table is valid for tiles of dash_attn_tile_size(S, D) and
 * deadlock free on P workgroups, DASH_ERR_TABLE if not; DASH_ERR_UNSUPPORTED
 * for more than 2^24 tasks, or tasks x passes. */
int dash_schedule_table_check(int S, int D, int mask, int G, int P, int items,
                              const int* item_offsets, const int* tasks);

/* Checks a table as dash_schedule_table_check does (on any grid wide enough
 * for its widest dispatch block) and writes its device form to `out` (host
 * memory; the caller copies it to device memory and passes that to
 * dash_attn_bwd_table).  Returns the bytes the device form takes (0 when the
 * table is invalid); with out == NULL only the size.  *status (may be NULL)
 * gets DASH_OK, the table's error, or DASH_ERR_WORKSPACE when out_bytes is
 * too small. */
size_t dash_schedule_table_pack(int S, int D, int mask, int G, int items, const int* item_offsets,
                                const int* tasks, void* out, size_t out_bytes, int* status);

/* dash_sim_run for a schedule given as a table (N tiles, G heads); the table
 * must be valid (else DASH_ERR_TABLE). */
int dash_sim_table(int mask, int N, int G, int groups, int P, int dispatch, double c_full,
                   double c_diag, double r, int items, const int* item_offsets, const int* tasks,
                   dash_sim_result* out);

/* Search over a family of block-wise lockstep walks for the shortest
 * simulated critical path (dynamic dispatch, `groups` groups on P
 * workgroups, weights as in dash_sim_run).  Candidates, in tie-break order:
 * each family kind that applies (SYMMETRIC, SHIFT, DESCENDING, ASCENDING,
 * PACKED; PACKED with G > 1 only for 256-key tiles),
 * units (chains, or symmetric pairs) in ascending then descending order, and
 * dispatch blocks of min(units, P), half that, and 1 consecutive units; dQ
 * tile (g, j) is reduced in the order (block, step at which the unit reaches
 * j, unit position).  The closed forms are members (e.g. SHIFT = shift kind,
 * ascending, one block), so the result is never worse than the best closed
 * form that runs on P workgroups, and the family reaches N > P, where the
 * shift family cannot run.  Candidates that fail dash_schedule_table_check
 * on P are skipped.  The packed kind (one order, `block` = its bins: the
 * workgroups one group gets, min(G * N, P / groups)) reaches beyond the
 * walks when equal chains leave workgroups idle at the end, e.g. a last
 * round of items for part of the grid.  Writes the winner (item_offsets:
 * G * N + 1 ints, tasks: 4 ints per task), family = {kind, order (0
 * ascending), block} (may be NULL) and its report (may be NULL). */
int dash_schedule_search(int S, int D, int mask, int G, int groups, int P, double c_full,
                         double c_diag, double r, int* items, int* item_offsets, int* tasks,
                         int* family, dash_sim_result* out);

/* The backward of dash_attn_bwd under a task table.  `table` is the device
 * copy (table_bytes bytes, 4-byte aligned) of what dash_schedule_table_pack
 * wrote for this S, D, mask and G = Hq / Hkv, with `items` items; the caller
 * owns it and must not change it while the call runs.  `grid` caps the
 * persistent workgroups (0 = dash_attn_bwd_grid_size; else 1 .. that), e.g.
 * to leave compute units to concurrent work; the launch uses min(grid,
 * B * Hkv * items).  The host checks sizes; the kernel checks the table's
 * header (shape, mask, passes, items, tasks) and that the launch is at least
 * as wide as the table's widest dispatch block; on a mismatch it computes
 * nothing and dash_attn_bwd_check reports DASH_ERR_TABLE.  Determinism
 * contract as for dash_attn_bwd: bitwise identical results for a fixed
 * table.  Workspace: dash_attn_bwd_workspace_size(..., DASH_SCHED_TABLE). */
int dash_attn_bwd_table(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int B, int Hq, int Hkv, int S, int D, int mask, const void* table,
                        size_t table_bytes, int items, int grid, void* workspace,
                        size_t workspace_bytes, void* stream);

/* The run phase of dash_attn_bwd_table alone, for callers that schedule or
 * time the two phases separately: dash_attn_bwd_prepare(..., DASH_SCHED_TABLE,
 * ...) on this workspace first, then this call (same arguments and checks as
 * dash_attn_bwd_table less o and lse; the preparation contract of
 * dash_attn_bwd_run, including DASH_ERR_NOT_PREPARED). */
int dash_attn_bwd_table_run(const void* q, const void* k, const void* v, const void* dout,
                            void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S, int D,
                            int mask, const void* table, size_t table_bytes, int items,
                            int grid, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DASH_ATTN_H */
