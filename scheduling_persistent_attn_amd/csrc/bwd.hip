// Deterministic attention backward for gfx950 (CDNA4).
//
// Kernels:
//   bwd_preprocess   per query row: -Dl = -rowsum(dO * O) and -lse/scale
//                    (padded to whole tiles with 0 and -inf), zeroing of the
//                    turn counters, the turn-wait counters and dispatch state.
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
// (query head, dQ tile, pass, wave slice): the reduction of rank r waits until
// the counter equals r, adds its partial into the fp32 accumulator in HBM,
// then publishes r + 1 (agent-scope, so the hand-off also works between the
// eight XCDs, whose L2 caches are not coherent with each other).
//
// Workgroup = T/32 waves; wave w owns keys [32w, 32w+32) of the key/value tile.
// Per task (KV tile i, Q tile j, query head h), per 32-row block of Q:
//   S - lse/scale = Q K^T  (accumulator starts at -lse/scale; A = Q rows, B = K rows)
//   dP - Dl       = dO V^T (accumulator starts at -Dl; B = V rows in registers)
//   P = exp2((S - lse/scale) * scale * log2e),  dS = P * (dP - Dl)
//   dV^T += dO^T P        A = dO^T (transposing LDS reads), B = P (registers)
//   dK^T += Q^T dS        A = Q^T  (transposing LDS reads), B = dS (registers)
//   dS -> LDS
// and per wave a 32-column slice of dQ = dS K with A = dS (LDS) and B = K^T
// fragments held in registers for the whole run of the KV tile (formed once by
// transposing LDS reads), followed by the ordered reduction.
// All products use v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32 accumulate).
// The 32x32 accumulator holds column n = lane % 32 and rows
// 8*(r/4) + 4*(lane/32) + r%4 in register r; a product whose contraction runs
// over those rows takes the accumulator (converted to bf16) directly as its B
// operand, provided its A operand enumerates the contraction index in the same
// permuted order -- which the transposing LDS reads provide.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "bwd_common.h"
#include "kernels.h"
#include "lds_layout.h"
#include "schedule.h"

namespace dash {

// ---------------------------------------------------------------------------
// Preprocess.  One row (b, h, s) of Dl per D/8 lanes; lanes reduce their
// 8-element partial dot products with a fixed butterfly.  Stores the values
// the main kernel's accumulators start from: -Dl, and -lse/scale (rows past
// S: 0 and -inf, so that P = 0 there).
__global__ __launch_bounds__(256) void bwd_preprocess(PreParams p) {
  // Rows are taken in the memory order of o and dout ([B, S, Hq, D]: the
  // rows of one block are contiguous), then the padding rows past S; each
  // row's value is stored at its [B*Hq][NT] position.  (Row counts fit in 32
  // bits: the host refuses sizes whose element offsets do not.)
  const int lpr = p.D / 8;
  const int rows_per_block = 256 / lpr;
  const int row = blockIdx.x * rows_per_block + threadIdx.x / lpr;
  const int sub = threadIdx.x % lpr;
  const int real = p.B * p.S * p.Hq;
  const int nrows = p.B * p.Hq * p.NT;
  float acc = 0.0f;
  int bh = 0, s = 0;
  if (row < real) {
    const int bs = row / p.Hq, h = row - bs * p.Hq;
    const int b = bs / p.S;
    s = bs - b * p.S;
    bh = b * p.Hq + h;
    const size_t off = (size_t)row * p.D + 8 * sub;
    const bf16x8 o = *reinterpret_cast<const bf16x8*>((const bf16*)p.o + off);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>((const bf16*)p.dout + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)o[e] * (float)g[e];
  } else if (row < nrows) {
    const int pad = p.NT - p.S, pr = row - real;
    bh = pr / pad;
    s = p.S + (pr - bh * pad);
  }
  for (int m = lpr / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < nrows && sub == 0) {
    const long long drow = (long long)bh * p.NT + s;
    p.delta[drow] = -acc;
    p.lse2[drow] = s < p.S ? -p.lse[(long long)bh * p.S + s] * p.inv_scale : -__builtin_inff();
  }
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nthreads = (long long)gridDim.x * blockDim.x;
  for (long long x = tid; x < p.n_counters; x += nthreads) p.counters[x] = 0;
  if (tid < 64) p.ctrl[tid] = 0;
  for (long long x = tid; x < 4LL * kWaitSlots; x += nthreads) p.waits[x] = 0;
  if (p.zero_dqacc) {
    f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    for (long long x = tid; x < p.n_dqacc / 4; x += nthreads)
      reinterpret_cast<f32x4*>(p.dqacc)[x] = z;
  }
}

// ---------------------------------------------------------------------------
// A task (KV tile i, Q tile j of T rows) is processed in passes of BQ query
// rows: QBP blocks of 32 rows, with BQ chosen so that the pass's dQ (BQ x D)
// splits into one 32 x 32 block per wave.  The operands a wave needs from its
// KV tile stay in registers for the whole run of the tile: the K and V rows
// it owns (B operands of S and dP) and the K^T fragments of its dQ feature
// block (B operand of dQ = dS K); the K tile passes through LDS once per run
// to form them.  The next pass's Q/dO rows and per-row -lse/scale, -Dl values
// are loaded into registers at the start of a pass and written into the other
// half of a double buffer in LDS late in it.  dS is triple-buffered: the dQ
// product of a slice, which needs every wave's dS, is formed two passes after
// that dS was written, so one workgroup barrier per pass suffices.  The
// ordered reduction of a slice is pipelined over the three passes that follow
// it: at the end of the first its turn (polled early in that pass) is checked
// and its partial sum loaded; in the second its product is added and stored
// (or, by the last contributor, written to dq in bf16); in the third its
// counter is published: after that pass's S/dP products when a task has four
// or more passes, else right after its opening barrier.  The round trips to the device-coherent
// level thus overlap with whole passes of computation.  The last pass of a KV
// tile's run finishes the open slices before the tile changes.
template <int D, int T, bool CAUSAL>
struct BwdCfg {
  static constexpr int NW = T / 32;      // waves; wave w owns keys [32w, 32w+32)
  static constexpr int DB = D / 32;      // 32-wide feature blocks
  static constexpr int QBP = NW / DB;    // 32-row blocks per pass
  static constexpr int BQ = 32 * QBP;    // query rows per pass
  static constexpr int NP = T / BQ;      // passes per task
  // Where a stored slice is published.  After the next pass's S/dP products
  // the stores have had the barrier and those products to be acknowledged,
  // instead of stalling the top of the pass; the price is a third of a pass
  // of hand-off delay, which tasks of four or more passes absorb (the next
  // contributor of a slice is a task later) and tasks of two do not.
  static constexpr bool PUBLISH_MID = NP >= 4;
  static constexpr int KBD = D / 16;     // k-blocks over the head dim
  static constexpr int KBT = T / 16;     // k-blocks over a tile of keys
  static constexpr int RBD = 2 * D;      // bytes per row of a Q/dO/K tile
  static constexpr int RBS = 2 * T;      // bytes per row of the dS block
  static constexpr int K_TILE = T * RBD, Q_TILE = BQ * RBD, S_TILE = BQ * RBS;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_Q = K_TILE;                 // + buf * Q_TILE
  static constexpr int OFF_DO = OFF_Q + 2 * Q_TILE;    // + buf * Q_TILE
  static constexpr int OFF_DS = OFF_DO + 2 * Q_TILE;   // + buf * S_TILE, 3 buffers
  static constexpr int OFF_LD = OFF_DS + 3 * S_TILE;   // [buf][-lse/scale | -Dl][BQ] fp32
  static constexpr int OFF_MISC = OFF_LD + 2 * 2 * 4 * BQ;
  static constexpr int LDS_BYTES = OFF_MISC + 16;
  static_assert(T >= D && NW % DB == 0 && T % BQ == 0, "tile shape");
  static_assert(RBD == 128 || RBD == 256, "head dim 64 or 128");
  static_assert(RBS == 128 || RBS == 256, "tile 64 or 128");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Per-lane LDS byte offsets.  The swizzle XORs a function of the row's low
// bits into the 16-byte slot index, and every access pattern of the kernel
// varies the slot index only in bits that this function leaves alone or in
// whole 16-row steps, so each pattern is one per-lane base XOR a constant (or
// plus a constant multiple of 16 rows, which the instruction's immediate
// offset absorbs).  Only the bases are kept in registers.
template <int D, int T>
struct LaneOffs {
  int a;      // 16-byte row reads of Q/dO/K: row c, chunk 2kb + hg is a ^ 32kb
  int s;      // 16-byte row reads of dS: row c, chunk 2kb + hg is s ^ 32kb
  int tq[2];  // transposing reads of Q/dO rows 8h8 + 4hg + (s16 >> 2), feature
              // block md: tq[h8] ^ 64md
  int kt[2];  // transposing reads of K rows 8hg + 4h4 + (s16 >> 2), features of
              // block db (+16kb rows: immediate offset)
  int wr;     // dS element writes of row 8(x >> 2) + 4hg + (x & 3), key 32w + c:
              // (wr ^ wx(x)) + wy(x)
  __device__ __forceinline__ int A(int kb) const { return a ^ (32 * kb); }
  __device__ __forceinline__ int S(int kb) const { return s ^ (32 * kb); }
  __device__ __forceinline__ int Tq(int md, int h8) const { return tq[h8] ^ (64 * md); }
  // constant parts of the dS write address of element x (see wr)
  static constexpr int wx(int x) {
    return T == 128 ? ((((x & 3) << 1) ^ ((x & 3) << 2) ^ (2 * (x >> 2))) << 4)
                    : ((8 * (x & 1) ^ 6 * ((x >> 1) & 1) ^ 3 * ((x >> 2) & 1)) << 4);
  }
  static constexpr int wy(int x) {
    return T == 128 ? (8 * (x >> 2) + (x & 3)) * 256 : (4 * (x >> 2) + ((x >> 1) & 1)) * 256;
  }
  __device__ __forceinline__ int W(int x) const { return (wr ^ wx(x)) + wy(x); }
};

// One wave's 32 x 32 slice of one pass of a dQ tile, and where it goes.
struct Slice {
  float* acc;      // fp32 accumulator of the slice (1024 floats)
  int* cnt;        // its turn counter
  int rank;        // position of this contribution in the tile's order
  int last;        // last contributor: writes bf16 dQ instead of the accumulator
  int dq_off;      // dq element of (slice row 0, feature 32*db + c)
  int rows_left;   // rows of the slice that exist: query rows < S, minus 1
};

// P = exp2((S - lse/scale) * scale * log2e) and dS = P * (dP - Dl), with the
// accumulators already holding S - lse/scale and dP - Dl (masked elements
// start at -inf, so P = 0 there); rounded to bf16 as the B operands of dV and
// dK.
__device__ __forceinline__ void softmax_block(const f32x16& sacc, const f32x16& dpacc, float scale_log2e,
                                              bf16x8* pb, bf16x8* dsb) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float pv = __builtin_amdgcn_exp2f(sacc[r] * scale_log2e);
    pb[r >> 3][r & 7] = (bf16)pv;
    dsb[r >> 3][r & 7] = (bf16)(pv * dpacc[r]);
  }
}

// This wave's dQ slice for one pass: 32 rows (block qg) x 32 features (block
// db), A = dS rows (LDS), B = K^T fragments (registers), accumulated onto c
// (the loaded partial sum of the earlier contributors, or zero).
template <int D, int T, bool CAUSAL>
__device__ __forceinline__ f32x16 dq_products(const char* lS, const LaneOffs<D, T>& o, int qg,
                                              const bf16x8* fkt, f32x16 c) {
  using C = BwdCfg<D, T, CAUSAL>;
  const int row0 = 32 * qg * C::RBS;
  bf16x8 fa[3];
  fa[0] = lds_read16(lS, o.S(0) + row0);
  fa[1] = lds_read16(lS, o.S(1) + row0);
#pragma unroll
  for (int kb = 0; kb < C::KBT; ++kb) {
    if (kb + 2 < C::KBT) fa[(kb + 2) % 3] = lds_read16(lS, o.S(kb + 2) + row0);
    c = mfma(fa[kb % 3], fkt[kb], c);
    __builtin_amdgcn_sched_barrier(0);  // reads stay ahead of their products
  }
  return c;
}

// dV^T += dO^T P and dK^T += Q^T dS over the 32 query rows of block m of the
// pass, fragments two steps ahead, with the block's dS element writes to lS
// spread over the steps (a scheduling barrier per step keeps that order).
template <int D, int T, bool CAUSAL>
__device__ __forceinline__ void dvdk_block(const char* lQ, const char* lO, const LaneOffs<D, T>& o, int m,
                                           const bf16x8* pb, const bf16x8* dsb, f32x16* dK, f32x16* dV,
                                           char* lS) {
  using C = BwdCfg<D, T, CAUSAL>;
  constexpr int X = 2 * C::DB;       // product steps
  constexpr int WPS = 16 / X;        // dS element writes per step
  bf16x8 fa[3], fb[3];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int md = x >> 1, kq = x & 1;
    const int base = (32 * m + 16 * kq) * C::RBD;
    fa[x] = lds_read_tr(lO, o.Tq(md, 0) + base, o.Tq(md, 1) + base);
    fb[x] = lds_read_tr(lQ, o.Tq(md, 0) + base, o.Tq(md, 1) + base);
  }
#pragma unroll
  for (int x = 0; x < X; ++x) {
    const int md = x >> 1, kq = x & 1;
    if (x + 2 < X) {
      const int md2 = (x + 2) >> 1, kq2 = (x + 2) & 1;
      const int base = (32 * m + 16 * kq2) * C::RBD;
      fa[(x + 2) % 3] = lds_read_tr(lO, o.Tq(md2, 0) + base, o.Tq(md2, 1) + base);
      fb[(x + 2) % 3] = lds_read_tr(lQ, o.Tq(md2, 0) + base, o.Tq(md2, 1) + base);
    }
    dV[md] = mfma(fa[x % 3], pb[kq], dV[md]);
    dK[md] = mfma(fb[x % 3], dsb[kq], dK[md]);
#pragma unroll
    for (int e = 0; e < WPS; ++e) {
      const int r = x * WPS + e;
      *reinterpret_cast<bf16*>(lS + o.W(r & 7) + (r >> 3) * 16 * C::RBS + 32 * m * C::RBS) = dsb[r >> 3][r & 7];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Accumulator loads of a slice (device-coherent): element r of lane l at
// float (r / 4) * 256 + 4 * l + r % 4, i.e. four fully coalesced 1 KB rows.
// With nbytes = 0 every load is out of range and returns zeros (used when
// there is no partial sum to add).
__device__ __forceinline__ f32x16 acc_load(float* acc, int nbytes, int lane) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(acc, 0, nbytes, 0x00020000);
  f32x16 v;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const f32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16 + q4 * 1024, 0, kSC1);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * q4 + e] = x[e];
  }
  return v;
}

// Second half of a slice's reduction: dq + old (the loaded partial sum, zero
// for rank 0), then store the new partial sum, or for the last contributor
// write dQ = scale * sum in bf16.  ATOMIC: unordered fp32 atomics instead.
template <bool ATOMIC>
__device__ __forceinline__ void acc_finish(const Slice& sl, f32x16 dq, int lane, int hg, int rs, float scale,
                                           bf16* gdq) {
  // rs is modified only by an empty asm statement below
  if constexpr (ATOMIC) {
    // element r of lane l at r*64 + l: each atomic instruction covers 64
    // consecutive floats
#pragma unroll
    for (int r = 0; r < 16; ++r) unsafeAtomicAdd(sl.acc + r * 64 + lane, dq[r]);
    return;
  } else {
    if (!sl.last) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(sl.acc, 0, 4096, 0x00020000);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 x = {dq[4 * q4], dq[4 * q4 + 1], dq[4 * q4 + 2], dq[4 * q4 + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(x, r, lane * 16 + q4 * 1024, 0, kSC1);
      }
    } else if (sl.rows_left >= 31) {
      asm volatile("" : "+s"(rs));  // keeps the row offsets from being hoisted out of the loop
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 8 * (r >> 2) + 4 * hg + (r & 3);
        gdq[sl.dq_off + ql * rs] = (bf16)(dq[r] * scale);
      }
    } else {
      // partial last tile: rows past S are not written
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 8 * (r >> 2) + 4 * hg + (r & 3);
        const int qc = min(ql, max(sl.rows_left, 0));
        const bf16 v = (bf16)(dq[r] * scale);
        if (ql <= sl.rows_left) gdq[sl.dq_off + qc * rs] = v;
      }
    }
  }
}

// One pass of the current task, plus two stages of the ordered reductions of
// earlier passes:
//   * slice `ld` (two passes back): its dQ product is formed from lS_ld on
//     top of the partial sum the previous pass loaded into dq_ld, then stored
//     (or, for the last contributor, written to dq) -- when ld_on;
//   * slice `prev` (the previous pass): its turn, polled at the start of the
//     pass, is checked at the end, then its partial sum is loaded into dq_ld
//     for the next pass (zeros when there is nothing to add);
//   * slice `rel` (stored at the end of the previous pass): with PUBLISH_MID
//     its counter is bumped after the S/dP products -- when rel_on.
// The partial-sum loads thus have most of a pass to arrive; the stores are
// acknowledged by the publish point (without PUBLISH_MID, the wait at the
// top of the next pass).  Everything from the first product to the dQ product has
// no branches, and scheduling barriers fix how far ahead of their products
// the fragment reads are issued (without a slice two passes back the dQ
// product is formed and dropped).  Writes dS of this pass into lS_cur.  When
// masked, elements with their bit set in zb[m] start at -inf (P = 0).
template <int D, int T, bool CAUSAL, bool ATOMIC>
__device__ __forceinline__ void pass_body(const char* lQ, const char* lO, const char* lL, char* lS_cur,
                                          const char* lS_ld, const LaneOffs<D, T>& o, int qg, int hg, int lane,
                                          float scale_log2e, bool masked, const unsigned* zb, const bf16x8* fk,
                                          const bf16x8* vB, const bf16x8* fkt, f32x16* dK, f32x16* dV,
                                          const Slice& ld, bool ld_on, f32x16& dq_ld, const Slice& prev,
                                          const Slice& rel, bool rel_on,
                                          const int* poll_ptr, int poll_expect, int polled, int acc_bytes,
                                          const BwdParams& p, int rs, bf16* gdq,
                                          const PassStage<D, BwdCfg<D, T, CAUSAL>::BQ, BwdCfg<D, T, CAUSAL>::NW>* stage,
                                          bool stage_on, char* st_q, char* st_o, char* st_l, int w) {
  using C = BwdCfg<D, T, CAUSAL>;
  constexpr int QBP = C::QBP;
  // ---- S and dP of the pass's 32-row blocks; the accumulators start at
  // -lse/scale and -Dl of their rows (rows 8(r/4) + 4hg + r%4)
  f32x16 sa[QBP], pa[QBP];
#pragma unroll
  for (int m = 0; m < QBP; ++m)
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const f32x4 l = *reinterpret_cast<const f32x4*>(lL + 4 * (32 * m + 8 * k4 + 4 * hg));
      const f32x4 d = *reinterpret_cast<const f32x4*>(lL + 4 * C::BQ + 4 * (32 * m + 8 * k4 + 4 * hg));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sa[m][4 * k4 + e] = l[e];
        pa[m][4 * k4 + e] = d[e];
      }
    }
  if (masked) {
#pragma unroll
    for (int m = 0; m < QBP; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[m][r] = ((zb[m] >> r) & 1u) ? -__builtin_inff() : sa[m][r];
  }
  {
    // fragments two k-blocks ahead of the products that use them
    bf16x8 fq[3][QBP], fd[3][QBP];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m = 0; m < QBP; ++m) {
        fq[kb][m] = lds_read16(lQ, o.A(kb) + 32 * m * C::RBD);
        fd[kb][m] = lds_read16(lO, o.A(kb) + 32 * m * C::RBD);
      }
#pragma unroll
    for (int kb = 0; kb < C::KBD; ++kb) {
      if (kb + 2 < C::KBD) {
#pragma unroll
        for (int m = 0; m < QBP; ++m) {
          fq[(kb + 2) % 3][m] = lds_read16(lQ, o.A(kb + 2) + 32 * m * C::RBD);
          fd[(kb + 2) % 3][m] = lds_read16(lO, o.A(kb + 2) + 32 * m * C::RBD);
        }
      }
#pragma unroll
      for (int m = 0; m < QBP; ++m) {
        sa[m] = mfma(fq[kb % 3][m], fk[kb], sa[m]);
        pa[m] = mfma(fd[kb % 3][m], vB[kb], pa[m]);
      }
      // (keeps the reads issued for kb + 2 ahead of this step's products;
      // without it the scheduler sinks each read next to its product and
      // every product waits for a full LDS round trip)
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- publish slice `rel`, whose partial-sum stores ended the previous
  // pass: since then only its four partial-sum loads, this pass's staging
  // loads and its turn poll were issued, so waiting until at most those are
  // outstanding means the stores are acknowledged.
  //   The count relies on this invariant: between the last store of `rel`
  // and this point each wave issues exactly 4 accumulator loads (acc_load,
  // always four b128 loads, out of range when nothing is added), 2 * KQ
  // staging loads plus one per-row value load (stage_load issues them
  // unconditionally, out of range when there is no next pass), and one turn
  // poll: 4 + 2 * KQ + 2 vector-memory operations, none of them conditional.
  // Vector-memory operations retire in issue order, so vmcnt <= that count
  // means every older operation, the stores included, has completed.  The
  // bit-identity tests at every workload size guard the count.
  if constexpr (!ATOMIC && C::PUBLISH_MID) {
    if (rel_on) {
      order_point();
      wait_vm<4 + 2 * PassStage<D, C::BQ, C::NW>::KQ + 2>();
      order_point();
      release(rel, lane);
    }
  }

  // ---- softmax: P and dS of this pass in bf16
  bf16x8 pb[QBP][2], dsb[QBP][2];
#pragma unroll
  for (int m = 0; m < QBP; ++m) softmax_block(sa[m], pa[m], scale_log2e, pb[m], dsb[m]);

  // ---- dV^T += dO^T P, dK^T += Q^T dS; dS -> LDS
#pragma unroll
  for (int m = 0; m < QBP; ++m) {
    dvdk_block<D, T, CAUSAL>(lQ, lO, o, m, pb[m], dsb[m], dK, dV, lS_cur);
  }

  // ---- dQ of the slice two passes back on top of its loaded partial sum
  // (late in the pass, so that the loads issued at the end of the previous
  // pass have had most of this pass to arrive)
  __builtin_amdgcn_sched_barrier(0);
  const f32x16 dq = dq_products<D, T, CAUSAL>(lS_ld, o, qg, fkt, dq_ld);

  // ---- the next pass's inputs into the other LDS buffer
  if (stage_on) stage_store<D, C::BQ, C::NW>(*stage, st_q, st_o, st_l, w, lane);

  // ---- turn of the previous slice (before the stores below are issued:
  // waiting for the poll then waits for nothing younger), the stores of the
  // slice two passes back, then the previous slice's partial sum: these four
  // loads are the last vector memory operations of the pass (the next pass's
  // barrier waits for everything before them)
  order_point();
  if constexpr (!ATOMIC) acquire(poll_ptr, poll_expect, polled, p.ctrl, p.spin_ticks, lane);
  order_point();
  if (ld_on) acc_finish<ATOMIC>(ld, dq, lane, hg, rs, p.scale, gdq);
  order_point();
  if constexpr (ATOMIC)
    dq_ld = f32x16{};
  else
    dq_ld = acc_load(prev.acc, acc_bytes, lane);
  order_point();
}

template <int D, int T, bool CAUSAL, int SCHED>
__global__ __attribute__((amdgpu_flat_work_group_size(2 * T, 2 * T)))
__attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_main(BwdParams p) {
  using C = BwdCfg<D, T, CAUSAL>;
  constexpr int BQ = C::BQ, NP = C::NP, QBP = C::QBP;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const char* const lK = smem + C::OFF_K;

  const int tid = threadIdx.x;
  // (the mask tells the compiler that w < NW, so the loaders need no bounds tests)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & (C::NW - 1);
  const int lane = tid & 63, c = lane & 31, hg = lane >> 5, g16 = lane >> 4, s16 = lane & 15;
  const int qg = w / C::DB, db = w % C::DB;  // this wave's dQ block within a pass
  constexpr int mask = CAUSAL ? MASK_CAUSAL : MASK_FULL;
  constexpr bool atomic_dq = SCHED == SCHED_ATOMIC;
  const int N = p.N, G = p.G, S = p.S;
  const int rsq = p.Hq * D;  // row stride of q / dout / dq
  bf16* const gdq = (bf16*)p.dq;

  // ---- per-lane LDS offsets ------------------------------------------------
  LaneOffs<D, T> o;
  o.a = lds_phys<C::RBD>(c, hg);
  o.s = lds_phys<C::RBS>(c, hg);
  // transposing reads of Q / dO: source lane s16 reads row 4hg + (s16 >> 2)
  // (+8 for the upper half), features 16(g16 & 1) + 4(s16 & 3) .. +3 of block 0
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8) {
    const int col = 16 * (g16 & 1) + 4 * (s16 & 3);
    o.tq[h8] = lds_phys<C::RBD>(8 * h8 + 4 * hg + (s16 >> 2), col >> 3) + 2 * (col & 7);
  }
  // transposing reads of K for dQ = dS K: keys 8hg + 4h4 + (s16 >> 2) of each
  // 16-key block, features of block db
#pragma unroll
  for (int h4 = 0; h4 < 2; ++h4) {
    const int col = 32 * db + 16 * (g16 & 1) + 4 * (s16 & 3);
    o.kt[h4] = lds_phys<C::RBD>(8 * hg + 4 * h4 + (s16 >> 2), col >> 3) + 2 * (col & 7);
  }
  // dS element writes: key 32w + c, row 4hg (+ the per-element constants)
  o.wr = lds_phys<C::RBS>(4 * hg, (32 * w + c) >> 3) + 2 * ((32 * w + c) & 7);
  // causal diagonal block: bit r set where key c comes after query row
  // 8(r >> 2) + 4hg + (r & 3) of the accumulator layout
  unsigned diag_bits = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) diag_bits |= (c > 8 * (r >> 2) + 4 * hg + (r & 3) ? 1u : 0u) << r;
  // loader: source (row, chunk) of the slot this lane fills in its first block
  int ldRow0, ldChunk0;
  lds_slot_source<C::RBD>(4 * w + (lane >> 4), lane & 15, &ldRow0, &ldChunk0);

  f32x16 dK[C::DB], dV[C::DB];
  // operands from the current KV tile, held for its whole run:
  bf16x8 fk[C::KBD];   // K rows 32w + c (B operand of S)
  bf16x8 vB[C::KBD];   // V rows 32w + c (B operand of dP)
  bf16x8 fkt[C::KBT];  // K^T, features of block db (B operand of dQ)

  // lane's byte offset of its 16-byte slot within a block of Q / dO rows
  const int voffQ = (ldRow0 * rsq + ldChunk0 * 8) * 2;
  PassStage<D, BQ, C::NW> stage;  // the next pass's inputs on their way to LDS

  int gp = 0;        // passes processed by this workgroup (selects the buffers)
  // reduction pipeline: prev = slice of the previous pass (dS in LDS), ld =
  // slice of two passes back (dS in LDS, partial sum loaded into dq_ld), rel
  // = slice whose stores are issued but whose counter is not yet bumped
  Slice prev = {}, ld = {}, rel = {};
  bool have_prev = false, have_ld = false, rel_pending = false;
  f32x16 dq_ld = {};
  int sb = 0;  // dS buffer of the current pass (of three)
  bool acc_tail = false;  // the last four vector memory operations are partial-sum loads
  bool first_item = true;
  if constexpr (SCHED == SCHED_TABLE) {
    if (!table_fits(p, NP, false)) {
      table_refused(p.ctrl);
      return;
    }
  }
  if (blockIdx.x == 0 && tid == 0) clock_stamp(p.ctrl + 8);
  for (;;) {
    __syncthreads();  // previous item's LDS use complete
    int* const misc = reinterpret_cast<int*>(smem + C::OFF_MISC);
    if (tid == 0) misc[0] = next_item(p.ctrl, p.total_items, first_item);
    first_item = false;
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(misc[0]);
    if (item >= p.total_items) {
      if (blockIdx.x == 0 && tid == 0) clock_stamp(p.ctrl + 12);
      break;
    }
    const int grp = item / p.items_per_group;
    const int local = item - grp * p.items_per_group;
    const int b = grp / p.Hkv, hk = grp - b * p.Hkv;
    const int first_task = item_first_task<SCHED>(p, local);
    const int len = item_tasks<SCHED>(p, mask, N, G, local);
    Task tn = item_task<SCHED>(p, mask, N, G, local, first_task, 0);
    stage_load<D, BQ, C::NW>(stage, p, T, b, hk * G + tn.g, tn.j, 0, true, voffQ, w, lane);
    stage_store<D, BQ, C::NW>(stage, smem + C::OFF_Q + (gp & 1) * C::Q_TILE, smem + C::OFF_DO + (gp & 1) * C::Q_TILE,
                              smem + C::OFF_LD + (gp & 1) * 2 * 4 * BQ, w, lane);

    for (int step = 0; step < len; ++step) {
      const Task t = tn;
      const int i = t.i, j = t.j, h = hk * G + t.g;
      const bool has_next = step + 1 < len;
      if (has_next) tn = item_task<SCHED>(p, mask, N, G, local, first_task, step + 1);
#ifdef DASH_TASK_TRACE
      const long long rec = SCHED == SCHED_TABLE ? (long long)grp * p.table_tasks + first_task + step
                                                 : (long long)item * p.trace_len + step;
      unsigned long long* const trec = trace_begin(p, rec, item, step, t.g, i, j, t.rank);
#endif
      if (t.seg_begin) {
        // new KV tile: K through LDS into this wave's K and K^T fragments, V
        // rows straight into registers
        __syncthreads();  // the K tile of the previous run is no longer read
        const int rs = p.Hkv * D;
        const int off = ((b * S + i * T) * p.Hkv + hk) * D;
        load_tile_async<D, T, C::NW>((const bf16*)p.k + off, rs, S - i * T, smem + C::OFF_K, w, ldRow0,
                                     ldChunk0);
        {
          const int nv = S - i * T;
          const int nbytes = nv <= 0 ? 0 : ((nv - 1) * rs + D) * 2;
          const __amdgpu_buffer_rsrc_t rv =
              __builtin_amdgcn_make_buffer_rsrc((void*)((const bf16*)p.v + off), 0, nbytes, 0x00020000);
#pragma unroll
          for (int kb = 0; kb < C::KBD; ++kb) {
            const f32x4 x =
                __builtin_amdgcn_raw_buffer_load_b128(rv, ((32 * w + c) * rs + 16 * kb + 8 * hg) * 2, 0, 0);
            vB[kb] = __builtin_bit_cast(bf16x8, x);
          }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // the K tile is in LDS
#pragma unroll
        for (int kb = 0; kb < C::KBD; ++kb) fk[kb] = lds_read16(lK, o.A(kb) + 32 * w * C::RBD);
#pragma unroll
        for (int kb = 0; kb < C::KBT; ++kb)
          fkt[kb] = lds_read_tr(lK, o.kt[0] + 16 * kb * C::RBD, o.kt[1] + 16 * kb * C::RBD);
        // the held fragments live in the accumulation registers (MFMA takes
        // its B operand from there), leaving the vector registers to the
        // per-pass work
#pragma unroll
        for (int kb = 0; kb < C::KBD; ++kb) asm volatile("" : "+a"(fk[kb]), "+a"(vB[kb]));
#pragma unroll
        for (int kb = 0; kb < C::KBT; ++kb) asm volatile("" : "+a"(fkt[kb]));
#pragma unroll
        for (int md = 0; md < C::DB; ++md) {
          dK[md] = f32x16{};
          dV[md] = f32x16{};
        }
      }
      const bool kv_tail = (i + 1) * T > S;
      const int key_local = 32 * w + c;
      const bool key_ok = i * T + key_local < S;
      const bool masked = (CAUSAL && i == j) || kv_tail;
      // this task's slices: pass hp is slice (tile * NP + hp) * NW + w
      const int slice0 = ((b * p.Hq + h) * N + j) * NP * C::NW + w;
      const bool last = t.rank == contributors(mask, N, j) - 1;
      const int r00 = j * T + 32 * qg;
      const int dq_off0 = (b * S + r00) * rsq + h * D + 32 * db + c;

      for (int hp = 0; hp < NP; ++hp, ++gp) {
        const int buf = gp & 1;
        const char* const lQ = smem + C::OFF_Q + buf * C::Q_TILE;
        const char* const lO = smem + C::OFF_DO + buf * C::Q_TILE;
        const char* const lL = smem + C::OFF_LD + buf * 2 * 4 * BQ;
        char* const lS_cur = smem + C::OFF_DS + sb * C::S_TILE;
        const int sb_ld = sb == 0 ? 1 : (sb == 1 ? 2 : 0);  // two passes back
        const char* const lS_ld = smem + C::OFF_DS + sb_ld * C::S_TILE;
        // re-materialise the offset bases each pass, so that the compiler
        // derives the per-access offsets here instead of keeping dozens of
        // them alive across the loop
        asm volatile("" : "+v"(o.a), "+v"(o.s), "+v"(o.tq[0]), "+v"(o.tq[1]), "+v"(o.kt[0]), "+v"(o.kt[1]),
                     "+v"(o.wr));
        // and keep the held K / V fragments in the accumulation registers
#pragma unroll
        for (int kb = 0; kb < C::KBD; ++kb) asm volatile("" : "+a"(fk[kb]), "+a"(vB[kb]));
#pragma unroll
        for (int kb = 0; kb < C::KBT; ++kb) asm volatile("" : "+a"(fkt[kb]));
        // this pass's inputs have arrived (the previous pass consumed them);
        // unless they are published mid-pass, so have the partial-sum stores
        // the previous pass ended with: wait for everything but its last
        // four operations, the partial-sum loads the dQ product waits for
        // itself.  (The atomic reference publishes nothing, so its
        // fire-and-forget atomics are not waited for here.)
        if constexpr (!atomic_dq) {
          if (!acc_tail)
            __builtin_amdgcn_s_waitcnt(0);
          else if constexpr (!C::PUBLISH_MID)
            wait_vm<4>();
        }
        // the previous pass's LDS writes (dS, the staged inputs) are complete
        // once lgkmcnt drains; no global memory is shared between the waves
        // here, so the barrier needs no memory fence
        order_point();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
        __builtin_amdgcn_s_barrier();
        order_point();
        if constexpr (!C::PUBLISH_MID) {
          if (rel_pending) {
            release(rel, lane);  // its stores completed at the wait above
            rel_pending = false;
          }
        }

        // the previous slice's turn counter is polled right after the
        // prefetch below (memory operations complete in issue order: the
        // prefetch, needed mid-pass, does not wait for the poll); without a
        // turn to take, poll a word that is always zero
        const bool need_turn = !atomic_dq && have_prev && prev.rank > 0;
        const int* const poll_ptr = need_turn ? prev.cnt : p.ctrl + 3;
        const int poll_expect = need_turn ? prev.rank : 0;
        const int acc_bytes = need_turn ? 4096 : 0;

        // prefetch the next pass into the other buffer (its readers finished
        // before the barrier above)
        const bool stage_next = hp + 1 < NP || has_next;
        {
          const bool same = hp + 1 < NP;
          stage_load<D, BQ, C::NW>(stage, p, T, b, same ? h : hk * G + tn.g, same ? j : tn.j, same ? hp + 1 : 0,
                                   stage_next, voffQ, w, lane);
        }
        order_point();
        const int polled = __hip_atomic_load(poll_ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        order_point();

        // this pass's slice
        Slice cur;
        {
          const int slice = slice0 + hp * C::NW;
          cur.acc = p.dqacc + slice * 1024;
          cur.cnt = p.counters + slice;
          cur.rank = t.rank;
          cur.last = last;
          cur.dq_off = dq_off0 + hp * BQ * rsq;
          cur.rows_left = S - 1 - r00 - hp * BQ;
        }

        unsigned zb[QBP];
#pragma unroll
        for (int m = 0; m < QBP; ++m) {
          const int qb = hp * QBP + m;  // 32-row block within the task
          unsigned z = 0;
          if (CAUSAL && i == j) z = w > qb ? 0xffffu : (w == qb ? diag_bits : 0u);
          if (kv_tail && !key_ok) z = 0xffffu;
          zb[m] = z;
        }
        pass_body<D, T, CAUSAL, atomic_dq>(lQ, lO, lL, lS_cur, lS_ld, o, qg, hg, lane, p.scale_log2e, masked, zb,
                                           fk, vB, fkt, dK, dV, ld, have_ld, dq_ld, prev, rel, rel_pending,
                                           poll_ptr, poll_expect,
                                           polled, acc_bytes, p, rsq, gdq, &stage, stage_next,
                                           smem + C::OFF_Q + (buf ^ 1) * C::Q_TILE,
                                           smem + C::OFF_DO + (buf ^ 1) * C::Q_TILE,
                                           smem + C::OFF_LD + (buf ^ 1) * 2 * 4 * BQ, w);
        acc_tail = true;
        if constexpr (C::PUBLISH_MID) rel_pending = false;  // published inside the pass body
        if (have_ld && !atomic_dq) {
          rel = ld;
          rel_pending = true;
        }
        ld = prev;
        have_ld = have_prev;

        if (hp == NP - 1 && t.seg_end) {
          // last pass of this KV tile's run: finish the two open slices now,
          // while the tile's fragments are still held
          __syncthreads();  // every wave's dS of this pass is in LDS
          // the previous pass's slice (partial sum already loaded): store it,
          // and publish it and the slice stored during this pass before
          // waiting for another turn (every chain of a lockstep group reaches
          // this point at once, so holding them here would close a cycle)
          const int sb_prev = sb == 0 ? 2 : sb - 1;
          if (have_ld) {
            const f32x16 dq = dq_products<D, T, CAUSAL>(smem + C::OFF_DS + sb_prev * C::S_TILE, o, qg, fkt, dq_ld);
            acc_finish<atomic_dq>(ld, dq, lane, hg, rsq, p.scale, gdq);
          }
          order_point();
          if constexpr (!atomic_dq) __builtin_amdgcn_s_waitcnt(0);
          order_point();
          if (!atomic_dq) {
            if (rel_pending) release(rel, lane);
            if (have_ld) release(ld, lane);
          }
          const bool ct = !atomic_dq && cur.rank > 0;
          if (ct) {
            const int pv = __hip_atomic_load(cur.cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            acquire(cur.cnt, cur.rank, pv, p.ctrl, p.spin_ticks, lane);
          }
          const f32x16 dq =
              dq_products<D, T, CAUSAL>(lS_cur, o, qg, fkt, acc_load(cur.acc, ct ? 4096 : 0, lane));
          acc_finish<atomic_dq>(cur, dq, lane, hg, rsq, p.scale, gdq);
          // release: all of this wave's accumulator stores acknowledged first
          order_point();
          if constexpr (!atomic_dq) __builtin_amdgcn_s_waitcnt(0);
          order_point();
          if (!atomic_dq) release(cur, lane);
          rel_pending = false;
          have_ld = false;
          have_prev = false;
          acc_tail = false;
        } else {
          prev = cur;
          have_prev = true;
        }
        sb = sb == 2 ? 0 : sb + 1;
      }

#ifdef DASH_TASK_TRACE
      trace_end(trec);
#endif
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

}

// ---------------------------------------------------------------------------
// Atomic reference only: dQ partial sums -> bf16 dq.  One thread per float of
// the accumulator, laid out as [tile][pass][wave slice][r][lane].
template <int D, int T>
__global__ __launch_bounds__(256) void bwd_finalize(FinParams p) {
  using C = BwdCfg<D, T, false>;
  constexpr int NW = C::NW, DB = C::DB, NP = C::NP;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)p.B * p.Hq * p.N * NP * NW * 16 * 64;
  if (idx >= total) return;
  // a launch that drained on its error flag (watchdog, or a run without its
  // prepare) leaves dq as it was
  if (__hip_atomic_load(p.ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  const int lane = (int)(idx % 64);
  long long rest = idx / 64;
  const int r = (int)(rest % 16);
  rest /= 16;
  const int w = (int)(rest % NW);
  rest /= NW;
  const int hp = (int)(rest % NP);
  rest /= NP;
  const int j = (int)(rest % p.N);
  const long long bh = rest / p.N;
  const int b = (int)(bh / p.Hq), h = (int)(bh % p.Hq);
  const int qg = w / DB, db = w % DB;
  const int ql = hp * C::BQ + 32 * qg + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  const int row = j * T + ql;
  if (row < p.S)
    ((bf16*)p.dq)[((size_t)((size_t)b * p.S + row) * p.Hq + h) * D + 32 * db + (lane & 31)] =
        (bf16)(p.dqacc[idx] * p.scale);
}

// ---------------------------------------------------------------------------
// The workspace of dash_attn_bwd_noalloc: a file-scope device array, one copy
// per GPU, held from the library's load until the process ends.  Host code
// never uses the array's name as an address: its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// kept, and only that address is passed to kernels.
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_workspace(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
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
    case SCHED_TABLE:
      hipLaunchKernelGGL((bwd_main<D, T, CAUSAL, SCHED_TABLE>), dim3(grid), dim3(2 * T), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_main(int D, int T, bool causal, const BwdParams& p, int grid,
                           hipStream_t s) {
  if (D == 64 && T == 64) return causal ? launch_sched<64, 64, true>(p.schedule, p, grid, s) : launch_sched<64, 64, false>(p.schedule, p, grid, s);
  if (D == 128 && T == 128) return causal ? launch_sched<128, 128, true>(p.schedule, p, grid, s) : launch_sched<128, 128, false>(p.schedule, p, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_finalize_atomic(int D, int T, const FinParams& p, hipStream_t s) {
  const long long total = (long long)p.B * p.Hq * p.N * T * D;  // accumulator floats
  const long long blocks = (total + 255) / 256;
  if (blocks < 1) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (D == 64 && T == 64) hipLaunchKernelGGL((bwd_finalize<64, 64>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else if (D == 128 && T == 128) hipLaunchKernelGGL((bwd_finalize<128, 128>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dash
