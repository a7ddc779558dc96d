// Deterministic attention backward for gfx950 (CDNA4).
//
// Kernels:
//   bwd_preprocess   Dl = rowsum(dO * O), lse2 = lse * log2(e) (padded to whole
//                    tiles), zeroing of the turn counters and dispatch state.
//   bwd_main         persistent backward: one workgroup per compute unit takes
//                    items (a key/value chain, or a symmetric pair of chains)
//                    from a device-wide counter and runs them tile by tile.
//   bwd_finalize     only for the non-deterministic atomic reference: dQ
//                    partial sums -> bf16.
//
// The method (DASH technical summary, sections 2.1-2.2): the dK/dV of a
// key/value tile stay in registers while one unit walks that tile's query
// tiles; each query tile's dQ is reduced across key/value tiles in a fixed
// order.  Here the fixed order is enforced with one turn counter per
// (query head, dQ tile, wave slice): the reduction of rank r waits until the
// counter equals r, adds its partial into the fp32 accumulator in HBM, then
// publishes r + 1 (agent-scope release/acquire, so the hand-off also works
// between the eight XCDs, whose L2 caches are not coherent with each other).
//
// Workgroup = T/32 waves; wave w owns keys [32w, 32w+32) of the key/value tile.
// Per task (KV tile i, Q tile j, query head h), per 32-row block mt of Q:
//   S    = Q K^T          A = Q rows (LDS),   B = K fragments (registers)
//   dP   = dO V^T         A = dO rows (LDS),  B = V fragments (registers)
//   P    = exp2(S*scale*log2e - lse*log2e),  dS = P * (dP - Dl)
//   dV^T += dO^T P        A = dO^T (LDS, transposed copy), B = P (registers)
//   dK^T += Q^T dS        A = Q^T  (LDS, transposed copy), B = dS (registers)
//   dS -> LDS
// then per wave a 32-column slice of dQ = dS K with A = dS (LDS) and B = K^T
// fragments (registers), followed by the ordered reduction.
// All products use v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32 accumulate).
// The 32x32 accumulator holds column n = lane % 32 and rows
// 8*(r/4) + 4*(lane/32) + r%4 in register r; a product whose contraction runs
// over those rows takes the accumulator (converted to bf16) directly as its B
// operand, provided its A operand enumerates the contraction index in the same
// permuted order -- which the transposed LDS copies provide with two 8-byte
// reads.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "schedule.h"

namespace dash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

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
// LDS tile layout.
//
// A tile is stored row-major in 256-byte "super-rows": a row of 256 bytes is
// one super-row; rows of 128 bytes are paired (row r is the half r & 1 of
// super-row r >> 1).  Each super-row holds 16 slots of 16 bytes and logical
// slot U of super-row R sits at slot U ^ sw(R).  The LDS of gfx950 serves
// 256 bytes per cycle from 64 four-byte banks; with
//   sw(R) = ((a << 1) ^ (a << 2)) ^ b,  a = R & 3,
//   b = (R >> 2) & 3 for 256-byte rows, (R >> 2) & 1 for 128-byte rows,
// both access shapes of the kernel are free of bank conflicts: 16-byte reads
// of one column in 16 consecutive rows, and the transposing 8-byte reads
// (ds_read_b64_tr_b16) of 4 consecutive rows x 64 bytes.  sw depends only on
// the low bits of the row, so moving by 16 rows is a constant offset.
__device__ __forceinline__ int sw16(int R, int row_bytes) {
  const int a = R & 3;
  const int b = row_bytes == 256 ? ((R >> 2) & 3) : ((R >> 2) & 1);
  return ((a << 1) ^ (a << 2)) ^ b;
}

// Byte offset of 16-byte chunk `chunk` of row `row` in a tile whose rows are
// row_bytes (128 or 256) long.
template <int RB>
__device__ __forceinline__ int phys(int row, int chunk) {
  static_assert(RB == 128 || RB == 256, "row length");
  if constexpr (RB == 256) {
    return row * 256 + ((chunk ^ sw16(row, 256)) << 4);
  } else {
    const int R = row >> 1;
    const int U = ((row & 1) << 3) | chunk;
    return R * 256 + ((U ^ sw16(R, 128)) << 4);
  }
}

// Inverse for the loader: physical slot `slot` of super-row R holds
// (row, chunk).
template <int RB>
__device__ __forceinline__ void slot_source(int R, int slot, int* row, int* chunk) {
  if constexpr (RB == 256) {
    *row = R;
    *chunk = slot ^ sw16(R, 256);
  } else {
    const int U = slot ^ sw16(R, 128);
    *row = 2 * R + (U >> 3);
    *chunk = U & 7;
  }
}

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

// ---------------------------------------------------------------------------
// Preprocess.  One row (b, h, s) of Dl per D/8 lanes; lanes reduce their
// 8-element partial dot products with a fixed butterfly.
__global__ __launch_bounds__(256) void bwd_preprocess(PreParams p) {
  const int lpr = p.D / 8;
  const int rows_per_block = 256 / lpr;
  const long long row = (long long)blockIdx.x * rows_per_block + threadIdx.x / lpr;
  const int sub = threadIdx.x % lpr;
  const long long nrows = (long long)p.B * p.Hq * p.NT;
  float acc = 0.0f;
  long long bh = 0;
  int s = 0;
  if (row < nrows) {
    bh = row / p.NT;
    s = (int)(row - bh * p.NT);
    if (s < p.S) {
      const long long b = bh / p.Hq, h = bh - b * p.Hq;
      const size_t off = ((size_t)(b * p.S + s) * p.Hq + h) * p.D + 8 * sub;
      const bf16x8 o = *reinterpret_cast<const bf16x8*>((const bf16*)p.o + off);
      const bf16x8 g = *reinterpret_cast<const bf16x8*>((const bf16*)p.dout + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)o[e] * (float)g[e];
    }
  }
  for (int m = lpr / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < nrows && sub == 0) {
    p.delta[row] = acc;
    p.lse2[row] = s < p.S ? p.lse[bh * p.S + s] * kLog2e : __builtin_inff();
  }
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nthreads = (long long)gridDim.x * blockDim.x;
  for (long long x = tid; x < p.n_counters; x += nthreads) p.counters[x] = 0;
  if (tid < 64) p.ctrl[tid] = 0;
  if (p.zero_dqacc) {
    f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    for (long long x = tid; x < p.n_dqacc / 4; x += nthreads)
      reinterpret_cast<f32x4*>(p.dqacc)[x] = z;
  }
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

// Turn wait with a watchdog.  Executed by a whole wave; lane 0 polls.  Returns
// false (and raises the workspace error flag) on timeout or if another wave
// already raised it.
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
  }
  ok = __shfl(ok, 0);
  order_point();
  return ok != 0;
}

// Asynchronous copy of ROWS rows of a bf16 tensor with row stride rs
// (elements) into an LDS tile, as 1 KB blocks (4 super-rows) of
// direct-to-LDS buffer loads; wave w issues blocks w, w + NW, ...  Rows at or
// past nvalid read as zero (the buffer's range check).  The slot a lane fills
// in block w + k*NW holds source row row0 + k*4*NW*RPS (RPS rows per
// super-row) and chunk chunk0, because the swizzle repeats every 16 (256-byte
// rows) or 8 (128-byte rows) super-rows; so one lane offset and a scalar
// per-block offset address every block.
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

// Asynchronous copy of 64 consecutive floats (a row range of the padded
// lse2 / Dl arrays) into LDS: one dword load of 64 lanes.
__device__ __forceinline__ void load_row_vec_async(const float* src, const char* dst, int lane) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, 256, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, lane * 4, 0, 0, 0);
}

// P = exp2(S * scale * log2e - lse * log2e) and dS = P * (dP - Dl) for one
// 32x32 accumulator block, rounded to bf16 as the B operands of dV and dK.
// MASKED: elements whose bit is set in zb are forced to P = 0.
template <bool MASKED>
__device__ __forceinline__ void softmax_block(const f32x16& sacc, const f32x16& dpacc, const f32x4* l2,
                                              const f32x4* dl, float scale_log2e, unsigned zb,
                                              bf16x8* pb, bf16x8* dsb) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float pv = __builtin_amdgcn_exp2f(sacc[r] * scale_log2e - l2[r >> 2][r & 3]);
    if constexpr (MASKED) pv = ((zb >> r) & 1u) ? 0.0f : pv;
    const float ds = pv * (dpacc[r] - dl[r >> 2][r & 3]);
    pb[r >> 3][r & 7] = (bf16)pv;
    dsb[r >> 3][r & 7] = (bf16)ds;
  }
}

// ---------------------------------------------------------------------------
// A task (KV tile i, Q tile j of T rows) is processed in passes of BQ = 64
// query rows.  Per pass the Q/dO rows, their lse2/Dl values and the dS block
// are BQ rows; the K and V tiles (T rows) stay in LDS for the whole run of the
// KV tile.  Q/dO/lse2/Dl are double-buffered: the next pass is copied into
// LDS while the current one computes.
template <int D, int T, bool CAUSAL>
struct BwdCfg {
  static constexpr int BQ = 64;          // query rows per pass
  static constexpr int NP = T / BQ;      // passes per task
  static constexpr int NW = T / 32;      // waves; wave w owns keys [32w, 32w+32)
  static constexpr int KBD = D / 16;     // k-blocks over the head dim
  static constexpr int KBT = T / 16;     // k-blocks over a tile of keys
  static constexpr int DB = D / 32;      // 32-wide feature blocks
  static constexpr int QBP = BQ / 32;    // 32-row blocks per pass
  static constexpr int MQ = QBP * DB / NW;  // dQ row blocks per wave and pass
  static constexpr int RBD = 2 * D;      // bytes per row of a Q/dO/K/V tile
  static constexpr int RBS = 2 * T;      // bytes per row of the dS block
  static constexpr int KV_TILE = T * RBD, Q_TILE = BQ * RBD;
  static constexpr int OFF_K = 0, OFF_V = KV_TILE;
  static constexpr int OFF_Q = 2 * KV_TILE;            // + buf * Q_TILE
  static constexpr int OFF_DO = OFF_Q + 2 * Q_TILE;    // + buf * Q_TILE
  static constexpr int OFF_DS = OFF_DO + 2 * Q_TILE;
  static constexpr int OFF_LD = OFF_DS + BQ * RBS;     // [buf][lse2 | Dl][BQ] fp32
  static constexpr int LDS_BYTES = OFF_LD + 2 * 2 * 4 * BQ;
  static_assert(T >= D && T % BQ == 0, "tile must be at least the head dim");
  static_assert(MQ >= 1 && (QBP * DB) % NW == 0, "dQ work split");
  static_assert(RBD == 128 || RBD == 256, "head dim 64 or 128");
  static_assert(RBS == 128 || RBS == 256, "tile 64 or 128");
};

template <int D, int T, bool CAUSAL, int SCHED>
__global__ __attribute__((amdgpu_flat_work_group_size(2 * T, 2 * T)))
__attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_main(BwdParams p) {
  using C = BwdCfg<D, T, CAUSAL>;
  constexpr int BQ = C::BQ, NP = C::NP;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const char* const lK = smem + C::OFF_K;
  const char* const lV = smem + C::OFF_V;
  char* const lS = smem + C::OFF_DS;

  const int tid = threadIdx.x;
  // (the mask tells the compiler that w < NW, so the loaders need no bounds tests)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & (C::NW - 1);
  const int lane = tid & 63, c = lane & 31, hg = lane >> 5, g16 = lane >> 4, s16 = lane & 15;
  const int qg = w / C::DB, db = w % C::DB;  // this wave's dQ block within a pass
  constexpr int mask = CAUSAL ? MASK_CAUSAL : MASK_FULL;
  constexpr bool atomic_dq = SCHED == SCHED_ATOMIC;
  const int N = p.N, G = p.G, S = p.S;

  // ---- per-lane LDS offsets, computed once ---------------------------------
  // 16-byte row reads: row c, chunk 2kb + hg (A fragments of S and dP from
  // Q/dO; B fragments from K/V rows 32w + c)
  int offA[C::KBD];
#pragma unroll
  for (int kb = 0; kb < C::KBD; ++kb) offA[kb] = phys<C::RBD>(c, 2 * kb + hg);
  // transposing reads of Q / dO for the A fragments of dK^T and dV^T:
  // source lane s16 reads row 4hg + (s16 >> 2) (+8 for the upper half),
  // features 32md + 16(g16 & 1) + 4(s16 & 3) .. +3
  int offT[C::DB][2];
#pragma unroll
  for (int md = 0; md < C::DB; ++md)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      const int col = 32 * md + 16 * (g16 & 1) + 4 * (s16 & 3);
      offT[md][h8] = phys<C::RBD>(8 * h8 + 4 * hg + (s16 >> 2), col >> 3) + 2 * (col & 7);
    }
  // transposing reads of K for the B fragments of dQ = dS K: keys
  // 8hg + 4h4 + (s16 >> 2) of each 16-key block, features of block db
  int offK[2];
#pragma unroll
  for (int h4 = 0; h4 < 2; ++h4) {
    const int col = 32 * db + 16 * (g16 & 1) + 4 * (s16 & 3);
    offK[h4] = phys<C::RBD>(8 * hg + 4 * h4 + (s16 >> 2), col >> 3) + 2 * (col & 7);
  }
  // A fragments of dQ: dS row c, chunk 2kb + hg
  int offS[C::KBT];
#pragma unroll
  for (int kb = 0; kb < C::KBT; ++kb) offS[kb] = phys<C::RBS>(c, 2 * kb + hg);
  // dS element writes: row 8((r >> 2) & 1) + 4hg + (r & 3), key 32w + c
  int offW[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int row = 8 * (x >> 2) + 4 * hg + (x & 3);
    const int key = 32 * w + c;
    offW[x] = phys<C::RBS>(row, key >> 3) + 2 * (key & 7);
  }
  // causal diagonal block: bit r set where key c comes after query row
  // 8(r >> 2) + 4hg + (r & 3) of the accumulator layout
  unsigned diag_bits = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) diag_bits |= (c > 8 * (r >> 2) + 4 * hg + (r & 3) ? 1u : 0u) << r;
  // loader: source (row, chunk) of the slot this lane fills in its first block
  int ldRow0, ldChunk0;
  slot_source<C::RBD>(4 * w + (lane >> 4), lane & 15, &ldRow0, &ldChunk0);

  f32x16 dK[C::DB], dV[C::DB];

  // Q, dO, lse2, Dl of rows [j*T + hp*BQ, +BQ) of head h into buffer buf
#define LOAD_PASS(b_, h_, j_, hp_, buf_)                                                     \
  do {                                                                                       \
    const int rs_ = p.Hq * D;                                                                \
    const int r0_ = (j_) * T + (hp_) * BQ;                                                   \
    const int off_ = (((b_) * S + r0_) * p.Hq + (h_)) * D;                                   \
    load_tile_async<D, BQ, C::NW>((const bf16*)p.q + off_, rs_, S - r0_,                     \
                                  smem + C::OFF_Q + (buf_) * C::Q_TILE, w, ldRow0, ldChunk0); \
    load_tile_async<D, BQ, C::NW>((const bf16*)p.dout + off_, rs_, S - r0_,                  \
                                  smem + C::OFF_DO + (buf_) * C::Q_TILE, w, ldRow0, ldChunk0); \
    const int row0_ = (((b_) * p.Hq + (h_)) * N + (j_)) * T + (hp_) * BQ;                    \
    if (w < 2)                                                                               \
      load_row_vec_async((w == 0 ? p.lse2 : p.delta) + row0_,                                \
                         smem + C::OFF_LD + ((buf_) * 2 + w) * 4 * BQ, lane);                \
  } while (0)

  int gp = 0;  // passes processed by this workgroup (selects the buffer)
  for (;;) {
    __syncthreads();  // previous item's LDS use complete
    if (tid == 0) {
      int it = atomicAdd(p.ctrl, 1);
      if (__hip_atomic_load(p.ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
        it = p.total_items;
      reinterpret_cast<int*>(lS)[0] = it;
    }
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(lS)[0]);
    if (item >= p.total_items) break;
    const int grp = item / p.items_per_group;
    const int local = item - grp * p.items_per_group;
    const int b = grp / p.Hkv, hk = grp - b * p.Hkv;
    const int len = item_len(mask, SCHED, N, G, local);
    __syncthreads();  // everyone has read the item index held in lS
    {
      const Task t0 = task_at(mask, SCHED, N, G, local, 0);
      LOAD_PASS(b, hk * G + t0.g, t0.j, 0, gp & 1);
    }

    for (int step = 0; step < len; ++step) {
      const Task t = task_at(mask, SCHED, N, G, local, step);
      const int i = t.i, j = t.j, h = hk * G + t.g;
      if (t.seg_begin) {
        __syncthreads();  // the K/V tiles of the previous segment are no longer read
        const int rs = p.Hkv * D;
        const int off = ((b * S + i * T) * p.Hkv + hk) * D;
        load_tile_async<D, T, C::NW>((const bf16*)p.k + off, rs, S - i * T, lK, w, ldRow0, ldChunk0);
        load_tile_async<D, T, C::NW>((const bf16*)p.v + off, rs, S - i * T, lV, w, ldRow0, ldChunk0);
#pragma unroll
        for (int md = 0; md < C::DB; ++md) {
          dK[md] = f32x16{};
          dV[md] = f32x16{};
        }
      }
      const bool diag = CAUSAL && i == j;
      const bool kv_tail = (i + 1) * T > S;
      const int key_local = 32 * w + c;
      const bool key_ok = i * T + key_local < S;

      for (int hp = 0; hp < NP; ++hp, ++gp) {
        const int buf = gp & 1;
        const char* const lQ = smem + C::OFF_Q + buf * C::Q_TILE;
        const char* const lO = smem + C::OFF_DO + buf * C::Q_TILE;
        const char* const lL = smem + C::OFF_LD + buf * 2 * 4 * BQ;
        const char* const lDl = lL + 4 * BQ;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // B1: this pass's Q/dO/lse2/Dl (and K/V) are in LDS

        // prefetch the next pass into the other buffer (its readers finished
        // before the previous pass's second barrier)
        if (hp + 1 < NP) {
          LOAD_PASS(b, h, j, hp + 1, buf ^ 1);
        } else if (step + 1 < len) {
          const Task tn = task_at(mask, SCHED, N, G, local, step + 1);
          LOAD_PASS(b, hk * G + tn.g, tn.j, 0, buf ^ 1);
        }

#pragma unroll 1
        for (int mt = 0; mt < C::QBP; ++mt) {
          const int qb = hp * C::QBP + mt;  // 32-row block within the task
          if (diag && w > qb) {
            // keys of this wave all come after these queries: dS block is zero
#pragma unroll
            for (int r = 0; r < 16; ++r)
              *reinterpret_cast<bf16*>(lS + offW[r & 7] + (r >> 3) * 16 * C::RBS + 32 * mt * C::RBS) =
                  (bf16)0.0f;
            continue;
          }
          f32x16 sacc = {}, dpacc = {};
          {
            bf16x8 fq[2], fd[2], fk[2], fv[2];
            fq[0] = lds_read16(lQ, offA[0] + 32 * mt * C::RBD);
            fd[0] = lds_read16(lO, offA[0] + 32 * mt * C::RBD);
            fk[0] = lds_read16(lK, offA[0] + 32 * w * C::RBD);
            fv[0] = lds_read16(lV, offA[0] + 32 * w * C::RBD);
#pragma unroll
            for (int kb = 0; kb < C::KBD; ++kb) {
              if (kb + 1 < C::KBD) {
                const int n = (kb + 1) & 1;
                fq[n] = lds_read16(lQ, offA[kb + 1] + 32 * mt * C::RBD);
                fd[n] = lds_read16(lO, offA[kb + 1] + 32 * mt * C::RBD);
                fk[n] = lds_read16(lK, offA[kb + 1] + 32 * w * C::RBD);
                fv[n] = lds_read16(lV, offA[kb + 1] + 32 * w * C::RBD);
              }
              sacc = mfma(fq[kb & 1], fk[kb & 1], sacc);
              dpacc = mfma(fd[kb & 1], fv[kb & 1], dpacc);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          f32x4 l2[4], dl[4];
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            l2[k4] = *reinterpret_cast<const f32x4*>(lL + 4 * (32 * mt + 8 * k4 + 4 * hg));
            dl[k4] = *reinterpret_cast<const f32x4*>(lDl + 4 * (32 * mt + 8 * k4 + 4 * hg));
          }
          bf16x8 pb[2], dsb[2];
          if ((diag && qb == w) || kv_tail) {
            // bit r of zb: element r is masked (key after query on the
            // diagonal block, or key past the sequence end)
            const unsigned zb = ((diag && qb == w) ? diag_bits : 0u) | ((kv_tail && !key_ok) ? 0xffffu : 0u);
            softmax_block<true>(sacc, dpacc, l2, dl, p.scale_log2e, zb, pb, dsb);
          } else {
            softmax_block<false>(sacc, dpacc, l2, dl, p.scale_log2e, 0u, pb, dsb);
          }
          {
            // dV^T += dO^T P and dK^T += Q^T dS over the 32 rows of block mt
            bf16x8 fa[2], fb[2];
            fa[0] = lds_read_tr(lO, offT[0][0] + 32 * mt * C::RBD, offT[0][1] + 32 * mt * C::RBD);
            fb[0] = lds_read_tr(lQ, offT[0][0] + 32 * mt * C::RBD, offT[0][1] + 32 * mt * C::RBD);
#pragma unroll
            for (int x = 0; x < 2 * C::DB; ++x) {
              const int md = x >> 1, kq = x & 1;
              if (x + 1 < 2 * C::DB) {
                const int md1 = (x + 1) >> 1, kq1 = (x + 1) & 1;
                const int base = (32 * mt + 16 * kq1) * C::RBD;
                fa[(x + 1) & 1] = lds_read_tr(lO, offT[md1][0] + base, offT[md1][1] + base);
                fb[(x + 1) & 1] = lds_read_tr(lQ, offT[md1][0] + base, offT[md1][1] + base);
              }
              dV[md] = mfma(fa[x & 1], pb[kq], dV[md]);
              dK[md] = mfma(fb[x & 1], dsb[kq], dK[md]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r)
            *reinterpret_cast<bf16*>(lS + offW[r & 7] + (r >> 3) * 16 * C::RBS + 32 * mt * C::RBS) =
                dsb[r >> 3][r & 7];
        }
        __syncthreads();  // B2: Q/dO/lse2/Dl reads of this pass done; dS complete

        // dQ slice of this wave for this pass: rows hp*BQ + [32*MQ*qg, +32*MQ),
        // features [32*db, +32)
        const int tile = (b * p.Hq + h) * N + j;
        const int slice = (tile * NP + hp) * C::NW + w;
        float* const acc = p.dqacc + slice * (C::MQ * 1024);
        int* const cnt = p.counters + slice;
        const int rank = t.rank;
        f32x16 dq[C::MQ];
#pragma unroll
        for (int m = 0; m < C::MQ; ++m) dq[m] = f32x16{};
        {
          bf16x8 fa[2][C::MQ], fb[2];
          const int qrow0 = 32 * qg * C::MQ * C::RBS;
#pragma unroll
          for (int m = 0; m < C::MQ; ++m) fa[0][m] = lds_read16(lS, offS[0] + qrow0 + 32 * m * C::RBS);
          fb[0] = lds_read_tr(lK, offK[0], offK[1]);
#pragma unroll
          for (int kb = 0; kb < C::KBT; ++kb) {
            if (kb + 1 < C::KBT) {
#pragma unroll
              for (int m = 0; m < C::MQ; ++m)
                fa[(kb + 1) & 1][m] = lds_read16(lS, offS[kb + 1] + qrow0 + 32 * m * C::RBS);
              fb[(kb + 1) & 1] = lds_read_tr(lK, offK[0] + 16 * (kb + 1) * C::RBD,
                                             offK[1] + 16 * (kb + 1) * C::RBD);
            }
#pragma unroll
            for (int m = 0; m < C::MQ; ++m) dq[m] = mfma(fa[kb & 1][m], fb[kb & 1], dq[m]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        if constexpr (atomic_dq) {
          // element r of row block m of lane l at (m*16 + r)*64 + l: each
          // atomic instruction covers 64 consecutive floats
#pragma unroll
          for (int m = 0; m < C::MQ; ++m)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              unsafeAtomicAdd(acc + (m * 16 + r) * 64 + lane, dq[m][r]);
        } else {
          const __amdgpu_buffer_rsrc_t racc =
              __builtin_amdgcn_make_buffer_rsrc(acc, 0, C::MQ * 4096, 0x00020000);
          const bool last = rank == contributors(mask, N, j) - 1;
          if (rank > 0) {
            wait_turn(cnt, rank, p.ctrl, p.spin_ticks, lane);
            f32x4 old[C::MQ][4];
#pragma unroll
            for (int m = 0; m < C::MQ; ++m)
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4)
                old[m][q4] = __builtin_amdgcn_raw_buffer_load_b128(
                    racc, (m * 4 * 64 + lane) * 16 + q4 * 1024, 0, kSC1);
#pragma unroll
            for (int m = 0; m < C::MQ; ++m)
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int e = 0; e < 4; ++e) dq[m][4 * q4 + e] = old[m][q4][e] + dq[m][4 * q4 + e];
          }
          if (!last) {
#pragma unroll
            for (int m = 0; m < C::MQ; ++m) {
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 x = {dq[m][4 * q4], dq[m][4 * q4 + 1], dq[m][4 * q4 + 2], dq[m][4 * q4 + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(x, racc, (m * 4 * 64 + lane) * 16 + q4 * 1024, 0, kSC1);
              }
            }
          } else {
            // final value: dQ = scale * sum, bf16
            bf16* const gdq = (bf16*)p.dq;
            const int rs = p.Hq * D;
            const int r0 = j * T + hp * BQ;
            const int base = (b * S + r0) * rs + h * D + 32 * db + c;
            const int last_row = S - 1 - r0;
            if (r0 + BQ <= S) {
#pragma unroll
              for (int m = 0; m < C::MQ; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const int ql = 32 * (qg * C::MQ + m) + 8 * (r >> 2) + 4 * hg + (r & 3);
                  gdq[base + ql * rs] = (bf16)(dq[m][r] * p.scale);
                }
            } else {
              // partial last tile: rows past S are not written
#pragma unroll
              for (int m = 0; m < C::MQ; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const int ql = 32 * (qg * C::MQ + m) + 8 * (r >> 2) + 4 * hg + (r & 3);
                  const int qc = min(ql, max(last_row, 0));
                  const bf16 v = (bf16)(dq[m][r] * p.scale);
                  if (ql <= last_row) gdq[base + qc * rs] = v;
                }
            }
          }
          // release: all of this wave's accumulator stores acknowledged first
          order_point();
          __builtin_amdgcn_s_waitcnt(0);
          order_point();
          if (lane == 0)
            __hip_atomic_store(cnt, rank + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }

      if (t.seg_end) {
        // dK = scale * dS^T Q, dV = P^T dO of key/value tile i, bf16
        if (i * T + key_local < S) {
          const int off = ((b * S + i * T + key_local) * p.Hkv + hk) * D;
          bf16* const gdk = (bf16*)p.dk;
          bf16* const gdv = (bf16*)p.dv;
#pragma unroll
          for (int md = 0; md < C::DB; ++md) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              bf16x4 xk, xv;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                xk[e] = (bf16)(dK[md][4 * q4 + e] * p.scale);
                xv[e] = (bf16)dV[md][4 * q4 + e];
              }
              const int d0 = 32 * md + 8 * q4 + 4 * hg;
              *reinterpret_cast<bf16x4*>(gdk + off + d0) = xk;
              *reinterpret_cast<bf16x4*>(gdv + off + d0) = xv;
            }
          }
        }
      }
    }
  }
#undef LOAD_PASS
}

// ---------------------------------------------------------------------------
// Atomic reference only: dQ partial sums -> bf16 dq.  One thread per float of
// the accumulator, laid out as [tile][pass][wave slice][row block m][r][lane].
template <int D, int T>
__global__ __launch_bounds__(256) void bwd_finalize(FinParams p) {
  using C = BwdCfg<D, T, false>;
  constexpr int NW = C::NW, DB = C::DB, MQ = C::MQ, NP = C::NP;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)p.B * p.Hq * p.N * NP * NW * MQ * 16 * 64;
  if (idx >= total) return;
  const int lane = (int)(idx % 64);
  long long rest = idx / 64;
  const int r = (int)(rest % 16);
  rest /= 16;
  const int m = (int)(rest % MQ);
  rest /= MQ;
  const int w = (int)(rest % NW);
  rest /= NW;
  const int hp = (int)(rest % NP);
  rest /= NP;
  const int j = (int)(rest % p.N);
  const long long bh = rest / p.N;
  const int b = (int)(bh / p.Hq), h = (int)(bh % p.Hq);
  const int qg = w / DB, db = w % DB;
  const int ql = hp * C::BQ + 32 * (qg * MQ + m) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  const int row = j * T + ql;
  if (row < p.S)
    ((bf16*)p.dq)[((size_t)((size_t)b * p.S + row) * p.Hq + h) * D + 32 * db + (lane & 31)] =
        (bf16)(p.dqacc[idx] * p.scale);
}

// ---------------------------------------------------------------------------
// Launch helpers

template <int D, int T, bool CAUSAL>
static int blocks_per_cu_impl() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, bwd_main<D, T, CAUSAL, SCHED_SHIFT>,
                                                   2 * T, 0) != hipSuccess)
    return 0;
  return nb;
}

int bwd_blocks_per_cu(int D, int T, bool causal) {
  if (D == 64 && T == 64) return causal ? blocks_per_cu_impl<64, 64, true>() : blocks_per_cu_impl<64, 64, false>();
  if (D == 64 && T == 128) return causal ? blocks_per_cu_impl<64, 128, true>() : blocks_per_cu_impl<64, 128, false>();
  if (D == 128 && T == 128) return causal ? blocks_per_cu_impl<128, 128, true>() : blocks_per_cu_impl<128, 128, false>();
  return 0;
}

int bwd_block_threads(int T) { return 2 * T; }

hipError_t launch_preprocess(const PreParams& p, hipStream_t s) {
  const int lpr = p.D / 8;
  const long long rows = (long long)p.B * p.Hq * p.NT;
  const long long rpb = 256 / lpr;
  long long blocks = (rows + rpb - 1) / rpb;
  if (blocks < 1) blocks = 1;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_preprocess, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D, int T, bool CAUSAL>
static hipError_t launch_sched(int sched, const BwdParams& p, int grid, hipStream_t s) {
  switch (sched) {
    case SCHED_NAIVE:
      hipLaunchKernelGGL((bwd_main<D, T, CAUSAL, SCHED_NAIVE>), dim3(grid), dim3(2 * T), 0, s, p);
      break;
    case SCHED_DESC:
      hipLaunchKernelGGL((bwd_main<D, T, CAUSAL, SCHED_DESC>), dim3(grid), dim3(2 * T), 0, s, p);
      break;
    case SCHED_SHIFT:
      hipLaunchKernelGGL((bwd_main<D, T, CAUSAL, SCHED_SHIFT>), dim3(grid), dim3(2 * T), 0, s, p);
      break;
    case SCHED_SYM:
      if constexpr (CAUSAL) {
        hipLaunchKernelGGL((bwd_main<D, T, CAUSAL, SCHED_SYM>), dim3(grid), dim3(2 * T), 0, s, p);
        break;
      }
      return hipErrorInvalidValue;
    case SCHED_ATOMIC:
      hipLaunchKernelGGL((bwd_main<D, T, CAUSAL, SCHED_ATOMIC>), dim3(grid), dim3(2 * T), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_main(int D, int T, bool causal, const BwdParams& p, int grid,
                           hipStream_t s) {
  if (D == 64 && T == 64) return causal ? launch_sched<64, 64, true>(p.schedule, p, grid, s) : launch_sched<64, 64, false>(p.schedule, p, grid, s);
  if (D == 64 && T == 128) return causal ? launch_sched<64, 128, true>(p.schedule, p, grid, s) : launch_sched<64, 128, false>(p.schedule, p, grid, s);
  if (D == 128 && T == 128) return causal ? launch_sched<128, 128, true>(p.schedule, p, grid, s) : launch_sched<128, 128, false>(p.schedule, p, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_finalize_atomic(int D, int T, const FinParams& p, hipStream_t s) {
  const long long total = (long long)p.B * p.Hq * p.N * T * D;  // accumulator floats
  const long long blocks = (total + 255) / 256;
  if (blocks < 1) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (D == 64 && T == 64) hipLaunchKernelGGL((bwd_finalize<64, 64>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else if (D == 64 && T == 128) hipLaunchKernelGGL((bwd_finalize<64, 128>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else if (D == 128 && T == 128) hipLaunchKernelGGL((bwd_finalize<128, 128>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dash
