// Device helpers shared by the persistent backward kernels: operand types,
// LDS fragment reads, and the ordered hand-off of dQ slices between
// workgroups (turn counters with a watchdog, the work-dispatch counter, the
// staged loads of each pass's inputs).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "lds_layout.h"
#include "schedule.h"

namespace dash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int s = 0; s < 8; ++s) z[s] = (bf16)0.0f;
  return z;
}

// ---------------------------------------------------------------------------
// LDS tiles use the swizzled layout of lds_layout.h: 16-byte row reads of one
// column in 16 consecutive rows and the transposing 8-byte reads of 4 rows x
// 64 bytes, or of two 4-row groups 8 rows apart x 32 bytes, are free of bank
// conflicts.

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ bf16x8 lds_read16(const char* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}
// two transposing reads -> one 16-element k-block operand fragment
__device__ __forceinline__ bf16x8 lds_read_tr(const char* base, int off0, int off1) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off0));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off1));
  bf16x8 a;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    a[s] = lo[s];
    a[s + 4] = hi[s];
  }
  return a;
}

// Element e of a packed bf16 fragment into LDS as it sits in its register
// half (no conversion: the high half goes out with ds_write_b16_d16_hi).
__device__ __forceinline__ void lds_write_bf16(char* at, const bf16x8& v, int e) {
  const unsigned pair = __builtin_bit_cast(uint4, v)[e >> 1];
  *reinterpret_cast<unsigned short*>(at) = (e & 1) ? (unsigned short)(pair >> 16) : (unsigned short)pair;
}

// ---------------------------------------------------------------------------
// The ordered hand-off of a dQ slice between workgroups.
//
// Every access to the fp32 dQ accumulator is a device-scope (sc1) buffer
// load or store, i.e. it is performed at the device's coherence point and
// never served from a stale line of this XCD's L2.  The hand-off therefore
// needs no cache-wide writeback or invalidate:
//   release: wait until this wave's sc1 stores are acknowledged (s_waitcnt),
//            then store rank + 1 into the turn counter (sc1);
//   acquire: poll the counter (sc1 loads) until it equals the rank; the
//            accumulator loads are issued only after the poll loop exits.
constexpr int kSC1 = 16;  // cache-policy operand of the buffer intrinsics: sc1

__device__ __forceinline__ void order_point() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// s_waitcnt for the vector-memory counter only: at most n of this wave's
// vector memory operations outstanding.  They complete in issue order, so
// this waits for everything but the last n issued.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // vmcnt[3:0] | expcnt[6:4] = 7 | lgkmcnt[11:8] = 15 | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Turn wait with a watchdog.  Executed by a whole wave; lane 0 polls.  Returns
// false (and raises the workspace error flag) on timeout or if another wave
// already raised it.  Only reached when the turn was not taken at the first
// check; each such wait is counted in the wave's slot of the wait counters,
// which follow the 64 control words in the workspace (one writer per slot, so
// the additions never contend).
__device__ __forceinline__ bool wait_turn(const int* cnt, int rank, int* ctrl,
                                          long long spin_ticks, int lane) {
  int ok = 1;
  if (lane == 0) {
    const long long t0 = wall_clock64();
    int polls = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != rank) {
      if ((++polls & 63) == 0) {
        if (__hip_atomic_load(ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
            wall_clock64() - t0 > spin_ticks) {
          ok = 0;
          break;
        }
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) {
      __hip_atomic_store(ctrl + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(ctrl + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int slot = (int)blockIdx.x * ((int)blockDim.x >> 6) + ((int)threadIdx.x >> 6);
    if (slot < kWaitSlots) {
      unsigned long long* st = reinterpret_cast<unsigned long long*>(ctrl + 64) + 4 * slot;
      const unsigned long long dt = (unsigned long long)(wall_clock64() - t0);
      __hip_atomic_fetch_add(st, 1ULL, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(st + 1, (unsigned long long)polls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(st + 2, dt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  ok = __shfl(ok, 0);
  order_point();
  return ok != 0;
}

// The shader clock (s_memtime) and the constant 100 MHz clock (s_memrealtime)
// into four control words; workgroup 0 stamps them when the persistent
// kernel starts (ctrl[8..11]) and when it leaves (ctrl[12..15]), and the
// ratio of the two intervals is the clock the compute unit ran at.
__device__ __forceinline__ void clock_stamp(int* at) {
  const unsigned long long t = clock64(), r = wall_clock64();
  unsigned long long* w = reinterpret_cast<unsigned long long*>(at);
  __hip_atomic_store(w, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(w + 1, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The next item index from the work-dispatch counter ctrl[0] (called by one
// thread per workgroup).  Each launch on a prepared workspace ends with one
// draw past the end per workgroup, so its draws are all below total + grid.  A
// launch that finds the counter at or past that on its first draw runs on a
// workspace the preprocess did not reset since the last launch (a run without
// its prepare): it raises the error flag ctrl[1] and the not-prepared mark
// ctrl[4], and every workgroup drains at once without touching the outputs.
// Once ctrl[1] is up (also by the watchdog) no further item is handed out.
__device__ __forceinline__ int next_item(int* ctrl, int total, bool first) {
  int it = atomicAdd(ctrl, 1);
  if (first && it >= total + (int)gridDim.x) {
    __hip_atomic_store(ctrl + 4, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ctrl + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (__hip_atomic_load(ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) it = total;
  return it;
}

// Asynchronous copy of ROWS rows of a bf16 tensor with row stride rs
// (elements) into an LDS tile, as 1 KB blocks (4 super-rows) of
// direct-to-LDS buffer loads; wave w issues blocks w, w + NW, ...  Rows at or
// past nvalid read as zero (the buffer's range check).  The slot a lane fills
// in block w + k*NW holds source row row0 + k*4*NW*RPS (RPS rows per
// super-row) and chunk chunk0, because the swizzle repeats every 16 (256-byte
// rows) or 8 (128-byte rows) super-rows; so one lane offset and a scalar
// per-block offset address every block.
// Whether a table schedule's header matches the launch: the shape, mask and
// passes per task it was checked for, its item and task counts, and a grid
// at least as wide as its widest dispatch block (the words are uniform).  A
// table in the per-head form also needs a kernel that writes per-head fp32
// dK/dV partials (`split_ok`) and a partial buffer with a slot per head.
__device__ __forceinline__ bool table_fits(const BwdParams& p, int passes, bool split_ok) {
  const unsigned* h = p.table;
  const bool split = (h[3] & kTableSplit) != 0;
  return h[0] == kTableMagic && h[1] == (unsigned)p.N && h[2] == (unsigned)p.G &&
         (h[3] & ~kTableSplit) == (unsigned)p.mask && h[4] == (unsigned)passes &&
         h[5] == (unsigned)p.items_per_group && h[6] <= gridDim.x && h[7] == (unsigned)p.table_tasks &&
         (!split || (split_ok && p.parts == p.G && p.dkv_part != nullptr));
}

// A table in the per-head form (its runs are one head's key/value tile).
__device__ __forceinline__ bool table_split(const BwdParams& p) { return (p.table[3] & kTableSplit) != 0; }

// A refused table: every workgroup leaves before touching any buffer, and
// workgroup 0 raises the error flag and the table mark (vector stores).
__device__ __forceinline__ void table_refused(int* ctrl) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    __hip_atomic_store(ctrl + 5, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ctrl + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Index of an item's first task in its group's task list (tables only) and
// its task count.
template <int SCHED>
__device__ __forceinline__ int item_first_task(const BwdParams& p, int item) {
  if constexpr (SCHED == SCHED_TABLE) return (int)p.table[kTableHeaderWords + item];
  return 0;
}
template <int SCHED>
__device__ __forceinline__ int item_tasks(const BwdParams& p, int mask, int N, int G, int item) {
  if constexpr (SCHED == SCHED_TABLE)
    return (int)(p.table[kTableHeaderWords + item + 1] - p.table[kTableHeaderWords + item]);
  return item_len(mask, SCHED, N, G, item);
}
// Task `step` of an item (first_task from item_first_task).
template <int SCHED>
__device__ __forceinline__ Task item_task(const BwdParams& p, int mask, int N, int G, int item, int first_task,
                                          int step) {
  if constexpr (SCHED == SCHED_TABLE) {
    const unsigned* w = p.table + table_task_words(p.items_per_group) + 2 * (first_task + step);
    return table_task(w[0], w[1]);
  }
  return task_at(mask, SCHED, N, G, item, step);
}

template <int D, int ROWS, int NW>
__device__ __forceinline__ void load_tile_async(const bf16* g, int rs, int nvalid, const char* dst,
                                                int w, int row0, int chunk0) {
  constexpr int BLK = ROWS * 2 * D / 1024;
  constexpr int RPS = 2 * D == 256 ? 1 : 2;  // rows per 256-byte super-row
  static_assert((2 * D == 256 && (4 * NW) % 16 == 0) || (2 * D == 128 && (4 * NW) % 8 == 0),
                "loader slot pattern must repeat every NW blocks");
  const int nbytes = nvalid <= 0 ? 0 : ((nvalid - 1) * rs + D) * 2;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)g, 0, nbytes, 0x00020000);
  const int voff = (row0 * rs + chunk0 * 8) * 2;
#pragma unroll
  for (int k = 0; k < (BLK + NW - 1) / NW; ++k) {
    const int blk = w + k * NW;
    if (blk < BLK)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + blk * 1024), 16, voff,
                                               k * 4 * NW * RPS * rs * 2, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// The inputs of one pass staged in registers on their way to LDS: this
// lane's 16-byte slots of the BQ rows of Q and dO (the slots the direct-to-LDS
// copies of load_tile_async fill) and one -lse/scale (wave 0) or -Dl (wave 1)
// value.  Loading into registers and writing LDS at the end of the pass keeps
// the LDS buffers out of the memory counter, so reads of the current buffer
// never wait for the next pass's copy.  Every wave issues the same 2 KQ + 1
// loads in every pass (out of range, returning zeros, when there is no next
// pass), which keeps the compiler's counter waits for older loads exact.
template <int D, int BQ, int NW>
struct PassStage {
  static constexpr int KQ = BQ * 2 * D / 1024 / NW;  // 1 KB blocks per wave and tensor
  f32x4 q[KQ], o[KQ];
  unsigned l;  // bit pattern of the fp32 value
};

template <int D, int BQ, int NW>
__device__ __forceinline__ void stage_load(PassStage<D, BQ, NW>& st, const BwdParams& p, int T, int b, int h,
                                           int j, int hp, bool valid, int voff, int w, int lane) {
  constexpr int RPS = 2 * D == 256 ? 1 : 2;  // rows per 256-byte super-row
  static_assert((BQ * 2 * D / 1024) % NW == 0, "whole blocks per wave");
  const int rs = p.Hq * D;
  const int r0 = j * T + hp * BQ;
  const int off = ((b * p.S + r0) * p.Hq + h) * D;
  const int nv = valid ? p.S - r0 : 0;
  const int nbytes = nv <= 0 ? 0 : ((nv - 1) * rs + D) * 2;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const bf16*)p.q + off), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const bf16*)p.dout + off), 0, nbytes, 0x00020000);
#pragma unroll
  for (int k = 0; k < PassStage<D, BQ, NW>::KQ; ++k) {
    const int soff = k * 4 * NW * RPS * rs * 2;
    st.q[k] = __builtin_amdgcn_raw_buffer_load_b128(rq, voff, soff, 0);
    st.o[k] = __builtin_amdgcn_raw_buffer_load_b128(ro, voff, soff, 0);
  }
  const int lrow = ((b * p.Hq + h) * p.N + j) * T + hp * BQ;
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((w == 0 ? p.lse2 : p.delta) + lrow), 0, valid ? 4 * BQ : 0, 0x00020000);
  st.l = __builtin_amdgcn_raw_buffer_load_b32(rl, lane * 4, 0, 0);
}

template <int D, int BQ, int NW>
__device__ __forceinline__ void stage_store(const PassStage<D, BQ, NW>& st, char* q_dst, char* o_dst, char* l_dst,
                                            int w, int lane) {
#pragma unroll
  for (int k = 0; k < PassStage<D, BQ, NW>::KQ; ++k) {
    const int off = (w + k * NW) * 1024 + lane * 16;
    *reinterpret_cast<f32x4*>(q_dst + off) = st.q[k];
    *reinterpret_cast<f32x4*>(o_dst + off) = st.o[k];
  }
  if (w < 2 && (BQ == 64 || lane < BQ)) *reinterpret_cast<unsigned*>(l_dst + w * 4 * BQ + lane * 4) = st.l;
}

// ---------------------------------------------------------------------------
// Pieces of the 256-key tile kernels (bwd_wide.hip, bwd_wide64.hip): the
// 16x16x32 product of the dQ slices, the dS block's layout and the slices
// themselves, all independent of the head dim.

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The dS block has 512-byte rows (32 slots of 16 bytes).  Slot U of row R sits
// at slot U ^ (R & 15): the 16-byte reads of one slot in 16 consecutive rows
// (the dQ product's A operand) then touch 16 different groups of four banks.
__device__ __forceinline__ int ds_phys(int row, int slot) {
  return row * 512 + ((slot ^ (row & 15)) << 4);
}

// One wave's 32 x 16 slice of one pass of a dQ tile, and where it goes.
struct WideSlice {
  float* acc;     // fp32 accumulator of the slice (512 floats)
  int* cnt;       // its turn counter
  int rank;       // position of this contribution in the tile's order
  int last;       // last contributor: writes bf16 dQ instead of the accumulator
  int dq_off;     // dq element of (slice row 0, feature 16w + s16)
  int rows_left;  // rows of the slice that exist: query rows < S, minus 1
};

struct DQ2 {
  f32x4 v[2];  // row blocks 0 and 1 (16 rows each)
};

// Accumulator loads of a slice (device-coherent): element r of row block rb
// of lane l at float rb*256 + 4l + r, i.e. two fully coalesced 1 KB rows.
// With nbytes = 0 both loads are out of range and return zeros.
__device__ __forceinline__ DQ2 wide_acc_load(float* acc, int nbytes, int lane) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(acc, 0, nbytes, 0x00020000);
  DQ2 v;
  v.v[0] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, kSC1);
  v.v[1] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16 + 1024, 0, kSC1);
  return v;
}

// Second half of a slice's reduction: store the new partial sum, or for the
// last contributor write dQ = scale * sum in bf16.  ATOMIC: unordered fp32
// atomics instead (element e of lane l at e*64 + l).
template <bool ATOMIC>
__device__ __forceinline__ void wide_acc_finish(const WideSlice& sl, const DQ2& dq, int lane, int rs, float scale,
                                                bf16* gdq, unsigned dq_bytes) {
  if constexpr (ATOMIC) {
#pragma unroll
    for (int e = 0; e < 8; ++e) unsafeAtomicAdd(sl.acc + e * 64 + lane, dq.v[e >> 2][e & 3]);
    return;
  } else {
    if (!sl.last) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(sl.acc, 0, 2048, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b128(dq.v[0], r, lane * 16, 0, kSC1);
      __builtin_amdgcn_raw_buffer_store_b128(dq.v[1], r, lane * 16 + 1024, 0, kSC1);
    } else {
      // dq rows 16(e/4) + 4(l/16) + e%4 of the slice, feature 16w + l%16; the
      // row stride stays opaque so that the per-element offsets are formed
      // here, not hoisted out of the loop into registers
      asm volatile("" : "+s"(rs));
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(gdq, 0, (int)dq_bytes, 0x00020000);
      const int vo = (sl.dq_off + 4 * (lane >> 4) * rs) * 2;
      if (sl.rows_left >= 31) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bf16 v = (bf16)(dq.v[e >> 2][e & 3] * scale);
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, vo,
                                                (16 * (e >> 2) + (e & 3)) * rs * 2, 0);
        }
      } else {
        // partial last tile: rows past S are not written
        const int r0 = 4 * (lane >> 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ql = 16 * (e >> 2) + r0 + (e & 3);
          const bf16 v = (bf16)(dq.v[e >> 2][e & 3] * scale);
          if (ql <= sl.rows_left)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, vo,
                                                  (16 * (e >> 2) + (e & 3)) * rs * 2, 0);
        }
      }
    }
  }
}

// Publishes rank + 1 on a slice's counter.  The caller has waited for this
// wave's accumulator stores (s_waitcnt) before.
template <class SliceT>
__device__ __forceinline__ void release(const SliceT& sl, int lane) {
  if (lane == 0) __hip_atomic_store(sl.cnt, sl.rank + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Blocks until *cnt equals expect, given a first poll result; the
// accumulator loads follow the acquire point.
__device__ __forceinline__ void acquire(const int* cnt, int expect, int polled, int* ctrl, long long spin_ticks,
                                        int lane) {
  if (__builtin_amdgcn_readfirstlane(polled) != expect) wait_turn(cnt, expect, ctrl, spin_ticks, lane);
  order_point();
}

}  // namespace dash
