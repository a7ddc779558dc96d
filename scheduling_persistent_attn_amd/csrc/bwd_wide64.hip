// Deterministic attention backward for gfx950, head dim 64, 256-key tiles.
//
// The method and hand-off protocol of bwd_wide.hip (head dim 128) at head dim
// 64.  A unit again holds the dK/dV of 256 keys on eight waves (two per SIMD;
// wave w owns keys [32w, 32w+32)), which at D = 64 costs only 64 registers
// per wave, so a pass covers 64 query rows: the same 48 matrix instructions
// per wave and pass as at D = 128, and the same bytes per FLOP (about 215
// FLOP per byte of Q/dO and partial-sum traffic, twice the 128-key tile's).
//
// Per pass of 64 query rows (two 32-row blocks) each wave computes, for its
// 32 keys,
//   S - lse/scale = Q K^T, dP - Dl = dO V^T, P, dS  (v_mfma_f32_32x32x16_bf16)
//   dV^T += dO^T P, dK^T += Q^T dS                  (v_mfma_f32_32x32x16_bf16)
// and writes dS to LDS.  The 64 x 64 dQ block of a pass is cut into eight
// 32-row x 16-feature slices, one per wave (row block w >> 2, features
// 16(w & 3) ..); a wave forms its slice dQ = dS K over all 256 keys
// (v_mfma_f32_16x16x32_bf16) one pass after the dS was written, holds the
// product in registers, and adds the loaded partial sum one pass later.  So
// the dS block of a pass is dead after the next pass and two dS buffers
// suffice (64 rows x 256 keys are 32 KiB each), which keeps the LDS within
// 160 KiB.  The turn of a slice is taken at the end of the pass after it and
// published in the third pass after it, as in bwd_wide.hip.
//
// Accumulator and operand layouts are those of bwd_wide.hip; LDS tiles of
// Q/dO/K have 128-byte rows in the swizzled layout of lds_layout.h, where
// moving by 16 rows adds 2048 bytes and by 32 rows 4096.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwd_common.h"
#include "kernels.h"
#include "lds_layout.h"
#include "schedule.h"

namespace dash {

struct Wide64Cfg {
  static constexpr int D = 64, T = 256;
  static constexpr int NW = 8;           // waves; wave w owns keys [32w, 32w+32)
  static constexpr int DB = D / 32;      // 32-wide feature blocks of dK/dV
  static constexpr int BQ = 64;          // query rows per pass
  static constexpr int RB = BQ / 32;     // 32-row blocks per pass
  static constexpr int NP = T / BQ;      // passes per task
  static constexpr int KBD = D / 16;     // 16-wide k-blocks over the head dim
  static constexpr int KBK = T / 32;     // 32-key k-steps of the dQ product
  static constexpr int KS = BQ / 16;     // 16-row k-steps of dV/dK
  static constexpr int SLICE = 512;      // floats per dQ slice (32 rows x 16 features)
  static constexpr int RBD = 2 * D;      // bytes per row of a Q/dO/K tile
  static constexpr int RBS = 2 * T;      // bytes per row of the dS block
  static constexpr int K_TILE = T * RBD, Q_TILE = BQ * RBD, S_TILE = BQ * RBS;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_Q = K_TILE;                // + buf * Q_TILE
  static constexpr int OFF_DO = OFF_Q + 2 * Q_TILE;   // + buf * Q_TILE
  static constexpr int OFF_DS = OFF_DO + 2 * Q_TILE;  // + buf * S_TILE, 2 buffers
  static constexpr int OFF_LD = OFF_DS + 2 * S_TILE;  // [buf][-lse/scale | -Dl][BQ] fp32
  static constexpr int OFF_MISC = OFF_LD + 2 * 2 * 4 * BQ;
  static constexpr int LDS_BYTES = OFF_MISC + 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(BQ * D == NW * SLICE, "one 32 x 16 dQ slice per wave and pass");
  static_assert(PassStage<D, BQ, NW>::KQ == 1, "counted wait below");
};

// Per-lane LDS byte offsets (the same access patterns as WideOffs in
// bwd_wide.hip, for 128-byte rows and two 32-row blocks per pass).
struct W64Offs {
  int a;      // 16-byte row reads of Q/dO/K: row c, chunk 2kb + hg is a ^ 32kb;
              // + 4096 per 32 rows
  int tq[2];  // transposing reads of Q/dO rows 8h8 + 4hg + (s16 >> 2), features
              // 16(g16 & 1) + 4(s16 & 3) of block md: tq[h8] ^ 64md; + 2048 per
              // 16-row k-step
  int kt[2];  // transposing reads of K rows 8g16 + 4h + (s16 >> 2), features
              // 16(w & 3) ..: + 4096 per 32-key k-step
  int sA;     // dQ A operand: dS row 32(w >> 2) + s16, keys 32kb + 8g16 ..:
              // sA ^ (kb << 6); + 8192 per 16 rows
  int wr;     // dS element writes of row 8(x >> 2) + 4hg + (x & 3), key 32w + c:
              // (wr ^ wx(x)) + wy(x); + 16384 per 32-row block
  __device__ __forceinline__ int A(int kb, int rb) const { return (a ^ (32 * kb)) + 4096 * rb; }
  __device__ __forceinline__ int Tq(int md, int h8) const { return tq[h8] ^ (64 * md); }
  __device__ __forceinline__ int SA(int kb, int r16) const { return (sA ^ (kb << 6)) + r16 * 8192; }
  static constexpr int wx(int x) { return ((8 * ((x >> 2) & 1)) | (x & 3)) << 4; }
  static constexpr int wy(int x) { return (8 * (x >> 2) + (x & 3)) * 512; }
  __device__ __forceinline__ int W(int x, int rb) const { return (wr ^ wx(x)) + wy(x) + 16384 * rb; }
};

// dQ slice of one pass: the wave's 32 rows x 16 features over the 256 keys;
// A = dS rows (LDS), B = K^T (transposing reads of the K tile), from zero.
__device__ __forceinline__ DQ2 w64_dq_products(const char* lS, const char* lK, const W64Offs& o) {
  using C = Wide64Cfg;
  DQ2 c;
  c.v[0] = f32x4{};
  c.v[1] = f32x4{};
  bf16x8 fa0[2], fa1[2], fb[2];
  fa0[0] = lds_read16(lS, o.SA(0, 0));
  fa1[0] = lds_read16(lS, o.SA(0, 1));
  fb[0] = lds_read_tr(lK, o.kt[0], o.kt[1]);
#pragma unroll
  for (int kb = 0; kb < C::KBK; ++kb) {
    if (kb + 1 < C::KBK) {
      fa0[(kb + 1) & 1] = lds_read16(lS, o.SA(kb + 1, 0));
      fa1[(kb + 1) & 1] = lds_read16(lS, o.SA(kb + 1, 1));
      fb[(kb + 1) & 1] = lds_read_tr(lK, o.kt[0] + (kb + 1) * 4096, o.kt[1] + (kb + 1) * 4096);
    }
    c.v[0] = mfma16(fa0[kb & 1], fb[kb & 1], c.v[0]);
    c.v[1] = mfma16(fa1[kb & 1], fb[kb & 1], c.v[1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  return c;
}

__device__ __forceinline__ DQ2 dq2_add(const DQ2& a, const DQ2& b) {
  DQ2 r;
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) r.v[k][e] = a.v[k][e] + b.v[k][e];
  return r;
}

// P = exp2((S - lse/scale) * scale * log2e), dS = P * (dP - Dl), rounded to
// bf16 as the B operands of dV and dK (two 16-row k-blocks per row block).
__device__ __forceinline__ void w64_softmax(const f32x16& sacc, const f32x16& dpacc, float scale_log2e,
                                            bf16x8* pb, bf16x8* dsb) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float pv = __builtin_amdgcn_exp2f(sacc[r] * scale_log2e);
    pb[r >> 3][r & 7] = (bf16)pv;
    dsb[r >> 3][r & 7] = (bf16)(pv * dpacc[r]);
  }
}

// dV^T += dO^T P and dK^T += Q^T dS over the 64 query rows of the pass (four
// 16-row k-steps), fragments one step ahead, with the dS element writes to
// lS spread over the steps.
__device__ __forceinline__ void w64_dvdk(const char* lQ, const char* lO, const W64Offs& o, const bf16x8* pb,
                                         const bf16x8* dsb, f32x16* dK, f32x16* dV, char* lS) {
  using C = Wide64Cfg;
  constexpr int X = C::DB * C::KS;     // product steps: (feature block, k-step)
  constexpr int WPS = 16 * C::RB / X;  // dS element writes per step
  bf16x8 fa[2], fb[2];
  fa[0] = lds_read_tr(lO, o.Tq(0, 0), o.Tq(0, 1));
  fb[0] = lds_read_tr(lQ, o.Tq(0, 0), o.Tq(0, 1));
#pragma unroll
  for (int x = 0; x < X; ++x) {
    const int ks = x % C::KS, md = x / C::KS;
    if (x + 1 < X) {
      const int ks2 = (x + 1) % C::KS, md2 = (x + 1) / C::KS;
      const int base = 2048 * ks2;
      fa[(x + 1) & 1] = lds_read_tr(lO, o.Tq(md2, 0) + base, o.Tq(md2, 1) + base);
      fb[(x + 1) & 1] = lds_read_tr(lQ, o.Tq(md2, 0) + base, o.Tq(md2, 1) + base);
    }
    dV[md] = mfma(fa[x & 1], pb[ks], dV[md]);
    dK[md] = mfma(fb[x & 1], dsb[ks], dK[md]);
#pragma unroll
    for (int e = 0; e < WPS; ++e) {
      const int q = x * WPS + e;  // element q & 15 of row block q >> 4
      const int r = q & 15, rb = q >> 4;
      lds_write_bf16(lS + o.W(r, rb), dsb[2 * rb + (r >> 3)], r & 7);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pass of the current task plus the stages of the ordered reductions of
// earlier passes: the slice of the previous pass (`pro`, its dS in the other
// LDS buffer) gets its product formed into registers and its turn taken, its
// partial sum loaded; the slice before it (`fin`: product held, partial sum
// loaded) is finished and stored; slice `rel` (stored at the end of the
// previous pass) is published after the S/dP products.
template <bool CAUSAL, bool ATOMIC>
__device__ __forceinline__ void w64_pass(const char* lQ, const char* lO, const char* lL, const char* lK,
                                         char* lS_cur, const char* lS_pro, const W64Offs& o, int lane, int w,
                                         float scale_log2e, bool masked, const unsigned* zb, const bf16x8* vB,
                                         f32x16* dK, f32x16* dV, bool pro_on, DQ2& h_pro, const WideSlice& fin,
                                         bool fin_on, const DQ2& h_fin, const DQ2& acc_fin, DQ2& acc_pro,
                                         const WideSlice& rel, bool rel_on, const int* poll_ptr, int poll_expect,
                                         int polled, int acc_bytes, const WideSlice& pro, const BwdParams& p,
                                         int rs, bf16* gdq, unsigned dq_bytes,
                                         const PassStage<64, 64, 8>* stage, bool stage_on, char* st_q, char* st_o,
                                         char* st_l) {
  using C = Wide64Cfg;
  const int hg = lane >> 5;
  // ---- S and dP of both row blocks; the accumulators start at -lse/scale
  // and -Dl of their rows
  f32x16 sa[C::RB], pa[C::RB];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const int row = 32 * rb + 8 * k4 + 4 * hg;
      const f32x4 l = *reinterpret_cast<const f32x4*>(lL + 4 * row);
      const f32x4 d = *reinterpret_cast<const f32x4*>(lL + 4 * C::BQ + 4 * row);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sa[rb][4 * k4 + e] = l[e];
        pa[rb][4 * k4 + e] = d[e];
      }
    }
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[rb][r] = ((zb[rb] >> r) & 1u) ? -__builtin_inff() : sa[rb][r];
    }
  }
  {
    const int kown = 4096 * w;  // this wave's K rows
    bf16x8 fq[2][C::RB], fd[2][C::RB], fk[2];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      fq[0][rb] = lds_read16(lQ, o.A(0, rb));
      fd[0][rb] = lds_read16(lO, o.A(0, rb));
    }
    fk[0] = lds_read16(lK, o.A(0, 0) + kown);
#pragma unroll
    for (int kb = 0; kb < C::KBD; ++kb) {
      if (kb + 1 < C::KBD) {
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          fq[(kb + 1) & 1][rb] = lds_read16(lQ, o.A(kb + 1, rb));
          fd[(kb + 1) & 1][rb] = lds_read16(lO, o.A(kb + 1, rb));
        }
        fk[(kb + 1) & 1] = lds_read16(lK, o.A(kb + 1, 0) + kown);
      }
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        sa[rb] = mfma(fq[kb & 1][rb], fk[kb & 1], sa[rb]);
        pa[rb] = mfma(fd[kb & 1][rb], vB[kb], pa[rb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- publish slice `rel`, whose partial-sum stores ended the previous
  // pass.  Since then this wave issued exactly: the two partial-sum loads of
  // `pro` (wide_acc_load, always two b128 loads), the next pass's staging
  // loads (stage_load: 2 * KQ = 2 tile loads and one per-row value load, all
  // unconditional) and one turn poll, i.e. 2 + 3 + 1 = 6 vector-memory
  // operations.  They retire in issue order, so once at most 6 are
  // outstanding the stores have completed.
  if constexpr (!ATOMIC) {
    if (rel_on) {
      order_point();
      wait_vm<6>();
      order_point();
      release(rel, lane);
    }
  }

  // ---- softmax, then dV^T += dO^T P, dK^T += Q^T dS; dS -> LDS
  bf16x8 pb[2 * C::RB], dsb[2 * C::RB];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) w64_softmax(sa[rb], pa[rb], scale_log2e, pb + 2 * rb, dsb + 2 * rb);
  // the dS element writes take the bf16 halves of these registers as they
  // are, instead of converting every element once more
#pragma unroll
  for (int k = 0; k < 2 * C::RB; ++k) asm volatile("" : "+v"(dsb[k]));
  w64_dvdk(lQ, lO, o, pb, dsb, dK, dV, lS_cur);

  // ---- dQ product of the previous pass's slice, from its dS (complete since
  // this pass's opening barrier)
  __builtin_amdgcn_sched_barrier(0);
  if (pro_on) h_pro = w64_dq_products(lS_pro, lK, o);

  // ---- the next pass's inputs into the other LDS buffer
  if (stage_on) stage_store<64, 64, 8>(*stage, st_q, st_o, st_l, w, lane);

  // ---- turn of `pro`, the stores of `fin`, then `pro`'s partial sum (the
  // last vector memory operations of the pass)
  order_point();
  if constexpr (!ATOMIC) acquire(poll_ptr, poll_expect, polled, p.ctrl, p.spin_ticks, lane);
  order_point();
  if (fin_on) wide_acc_finish<ATOMIC>(fin, dq2_add(acc_fin, h_fin), lane, rs, p.scale, gdq, dq_bytes);
  order_point();
  if constexpr (ATOMIC) {
    acc_pro.v[0] = f32x4{};
    acc_pro.v[1] = f32x4{};
  } else {
    acc_pro = wide_acc_load(pro.acc, acc_bytes, lane);
  }
  order_point();
}

template <bool CAUSAL, int SCHED>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512)))
__attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_main_wide64(BwdParams p) {
  using C = Wide64Cfg;
  constexpr int T = C::T, D = C::D, BQ = C::BQ, NP = C::NP;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const char* const lK = smem + C::OFF_K;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & (C::NW - 1);
  const int lane = tid & 63, c = lane & 31, hg = lane >> 5, g16 = lane >> 4, s16 = lane & 15;
  const int qr = w >> 2, fd = w & 3;  // the wave's dQ slice: row block, feature block
  constexpr int mask = CAUSAL ? MASK_CAUSAL : MASK_FULL;
  constexpr bool atomic_dq = SCHED == SCHED_ATOMIC;
  const int N = p.N, G = p.G, S = p.S;
  const int rsq = p.Hq * D;  // row stride of q / dout / dq
  bf16* const gdq = (bf16*)p.dq;
  // bytes of dq (below 2^32: the host keeps element offsets below 2^31)
  const unsigned dq_bytes = (unsigned)p.B * (unsigned)S * (unsigned)p.Hq * (unsigned)(2 * D);

  // ---- per-lane LDS offsets
  W64Offs o;
  o.a = lds_phys<C::RBD>(c, hg);
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8) {
    const int col = 16 * (g16 & 1) + 4 * (s16 & 3);
    o.tq[h8] = lds_phys<C::RBD>(8 * h8 + 4 * hg + (s16 >> 2), col >> 3) + 2 * (col & 7);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = 16 * fd + 4 * (s16 & 3);
    o.kt[h] = lds_phys<C::RBD>(8 * g16 + 4 * h + (s16 >> 2), col >> 3) + 2 * (col & 7);
  }
  o.sA = ds_phys(32 * qr + s16, g16);
  o.wr = ds_phys(4 * hg, (32 * w + c) >> 3) + 2 * (c & 7);
  // causal diagonal block: bit r set where key c comes after query row
  // 8(r >> 2) + 4hg + (r & 3)
  unsigned diag_bits = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) diag_bits |= (c > 8 * (r >> 2) + 4 * hg + (r & 3) ? 1u : 0u) << r;
  int ldRow0, ldChunk0;
  lds_slot_source<C::RBD>(4 * w + (lane >> 4), lane & 15, &ldRow0, &ldChunk0);

  f32x16 dK[C::DB], dV[C::DB];
  bf16x8 vB[C::KBD];  // V rows 32w + c (B operand of dP), held for the tile's run

  const int voffQ = (ldRow0 * rsq + ldChunk0 * 8) * 2;
  PassStage<D, BQ, C::NW> stage;

  int gp = 0;
  // reduction pipeline: pro = slice of the previous pass (dS in LDS), fin =
  // slice of two passes back (product in h_fin, partial sum in acc_fin), rel
  // = slice stored at the end of the previous pass, not yet published
  WideSlice pro = {}, fin = {}, rel = {};
  bool have_pro = false, have_fin = false, rel_pending = false;
  DQ2 h_fin = {}, acc_fin = {};
  bool acc_tail = false;  // the last two vector memory operations are partial-sum loads
  bool first_item = true;
  if constexpr (SCHED == SCHED_TABLE) {
    if (!table_fits(p, NP, true)) {
      table_refused(p.ctrl);
      return;
    }
  }
  // a table in the per-head form: each run's dK/dV go out as its head's fp32
  // partial, summed by bwd_dkv_finalize, which looks for this mark
  const bool split = SCHED == SCHED_TABLE && table_split(p);
  if (split && blockIdx.x == 0 && tid == 0)
    __hip_atomic_store(p.ctrl + 6, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (blockIdx.x == 0 && tid == 0) clock_stamp(p.ctrl + 8);
  // the older wave of each SIMD's pair (waves 0-3) issues first: the
  // hardware already favours it, and letting it run further ahead gets its
  // memory requests out earlier (measured 0.5-3 % faster on the best
  // schedules; raising waves 4-7 instead was slower)
  if (w < C::NW / 2) __builtin_amdgcn_s_setprio(3);
  for (;;) {
    __syncthreads();
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
    // this item's part of the group's query heads and its base item
    const int part = local / p.base_items;
    const int base = local - part * p.base_items;
    const int Gp = p.Gp;
    const int h0 = hk * G + part * Gp;  // first query head of the part
    const int first_task = item_first_task<SCHED>(p, base);
    const int len = item_tasks<SCHED>(p, mask, N, Gp, base);
    Task tn = item_task<SCHED>(p, mask, N, Gp, base, first_task, 0);
    stage_load<D, BQ, C::NW>(stage, p, T, b, h0 + tn.g, tn.j, 0, true, voffQ, w, lane);
    stage_store<D, BQ, C::NW>(stage, smem + C::OFF_Q + (gp & 1) * C::Q_TILE, smem + C::OFF_DO + (gp & 1) * C::Q_TILE,
                              smem + C::OFF_LD + (gp & 1) * 2 * 4 * BQ, w, lane);

    for (int step = 0; step < len; ++step) {
      const Task t = tn;
      const int i = t.i, j = t.j, h = h0 + t.g;
      const bool has_next = step + 1 < len;
      if (has_next) tn = item_task<SCHED>(p, mask, N, Gp, base, first_task, step + 1);
#ifdef DASH_TASK_TRACE
      const long long rec = SCHED == SCHED_TABLE ? (long long)grp * p.table_tasks + first_task + step
                                                 : (long long)item * p.trace_len + step;
      unsigned long long* const trec = trace_begin(p, rec, item, step, h - hk * G, i, j, t.rank);
#endif
      if (t.seg_begin) {
        // new KV tile: K into LDS, V rows of this wave's keys into registers
        __syncthreads();  // the K tile of the previous run is no longer read
        const int rs = p.Hkv * D;
        const int off = ((b * S + i * T) * p.Hkv + hk) * D;
        load_tile_async<D, T, C::NW>((const bf16*)p.k + off, rs, S - i * T, smem + C::OFF_K, w, ldRow0, ldChunk0);
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
      const int r00 = j * T + 32 * qr;  // first query row of the wave's slices
      const int dq_off0 = (b * S + r00) * rsq + h * D + 16 * fd + s16;

      for (int hp = 0; hp < NP; ++hp, ++gp) {
        const int buf = gp & 1;
        const char* const lQ = smem + C::OFF_Q + buf * C::Q_TILE;
        const char* const lO = smem + C::OFF_DO + buf * C::Q_TILE;
        const char* const lL = smem + C::OFF_LD + buf * 2 * 4 * BQ;
        char* const lS_cur = smem + C::OFF_DS + buf * C::S_TILE;
        const char* const lS_pro = smem + C::OFF_DS + (buf ^ 1) * C::S_TILE;
        asm volatile("" : "+v"(o.a), "+v"(o.tq[0]), "+v"(o.tq[1]), "+v"(o.kt[0]), "+v"(o.kt[1]), "+v"(o.sA),
                     "+v"(o.wr));
        // the partial-sum stores the previous pass ended with are published
        // mid-pass; only a pass that follows no pass body waits for all
        if constexpr (!atomic_dq) {
          if (!acc_tail) __builtin_amdgcn_s_waitcnt(0);
        }
        order_point();
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
        __builtin_amdgcn_s_barrier();
        order_point();

        const bool need_turn = !atomic_dq && have_pro && pro.rank > 0;
        const int* const poll_ptr = need_turn ? pro.cnt : p.ctrl + 3;
        const int poll_expect = need_turn ? pro.rank : 0;
        const int acc_bytes = need_turn ? 2048 : 0;

        const bool stage_next = hp + 1 < NP || has_next;
        {
          const bool same = hp + 1 < NP;
          stage_load<D, BQ, C::NW>(stage, p, T, b, same ? h : h0 + tn.g, same ? j : tn.j, same ? hp + 1 : 0,
                                   stage_next, voffQ, w, lane);
        }
        order_point();
        const int polled = __hip_atomic_load(poll_ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        order_point();

        WideSlice cur;
        {
          const int slice = slice0 + hp * C::NW;
          cur.acc = p.dqacc + slice * C::SLICE;
          cur.cnt = p.counters + slice;
          cur.rank = t.rank;
          cur.last = last;
          cur.dq_off = dq_off0 + hp * BQ * rsq;
          cur.rows_left = S - 1 - r00 - hp * BQ;
        }

        // masks of the two row blocks: query rows 64hp + 32rb + .., keys 32w + c
        unsigned zb[C::RB];
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          const int qb = 2 * hp + rb;  // 32-row block of the query tile
          unsigned z = 0;
          if (CAUSAL && i == j) z = w > qb ? 0xffffu : (w == qb ? diag_bits : 0u);
          if (kv_tail && !key_ok) z = 0xffffu;
          zb[rb] = z;
        }
        DQ2 h_pro = {}, acc_pro;
        w64_pass<CAUSAL, atomic_dq>(lQ, lO, lL, lK, lS_cur, lS_pro, o, lane, w, p.scale_log2e, masked, zb, vB, dK,
                                    dV, have_pro, h_pro, fin, have_fin, h_fin, acc_fin, acc_pro, rel, rel_pending,
                                    poll_ptr, poll_expect, polled, acc_bytes, pro, p, rsq, gdq, dq_bytes, &stage,
                                    stage_next, smem + C::OFF_Q + (buf ^ 1) * C::Q_TILE,
                                    smem + C::OFF_DO + (buf ^ 1) * C::Q_TILE,
                                    smem + C::OFF_LD + (buf ^ 1) * 2 * 4 * BQ);
        acc_tail = true;
        rel_pending = false;  // published inside the pass body
        if (have_fin && !atomic_dq) {
          rel = fin;
          rel_pending = true;
        }
        fin = pro;
        have_fin = have_pro;
        h_fin = h_pro;
        acc_fin = acc_pro;

        if (hp == NP - 1 && t.seg_end) {
          // last pass of this KV tile's run: finish the open slices while the
          // K tile is still in LDS
          __syncthreads();  // every wave's dS of this pass is in LDS
          const DQ2 h_cur = w64_dq_products(lS_cur, lK, o);
          if (have_fin) wide_acc_finish<atomic_dq>(fin, dq2_add(acc_fin, h_fin), lane, rsq, p.scale, gdq, dq_bytes);
          order_point();
          if constexpr (!atomic_dq) __builtin_amdgcn_s_waitcnt(0);
          order_point();
          if (!atomic_dq) {
            if (rel_pending) release(rel, lane);
            if (have_fin) release(fin, lane);
          }
          const bool ct = !atomic_dq && cur.rank > 0;
          if (ct) {
            const int pv = __hip_atomic_load(cur.cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            acquire(cur.cnt, cur.rank, pv, p.ctrl, p.spin_ticks, lane);
          }
          DQ2 acc_cur;
          if constexpr (atomic_dq) {
            acc_cur.v[0] = f32x4{};
            acc_cur.v[1] = f32x4{};
          } else {
            acc_cur = wide_acc_load(cur.acc, ct ? 2048 : 0, lane);
          }
          wide_acc_finish<atomic_dq>(cur, dq2_add(acc_cur, h_cur), lane, rsq, p.scale, gdq, dq_bytes);
          order_point();
          if constexpr (!atomic_dq) __builtin_amdgcn_s_waitcnt(0);
          order_point();
          if (!atomic_dq) release(cur, lane);
          rel_pending = false;
          have_fin = false;
          have_pro = false;
          acc_tail = false;
        } else {
          pro = cur;
          have_pro = true;
        }
      }

#ifdef DASH_TASK_TRACE
      trace_end(trec);
#endif
      if (t.seg_end && (SCHED == SCHED_TABLE ? split : p.parts > 1)) {
        // this part's fp32 dK/dV of key/value tile i (unscaled), summed over
        // the parts by bwd_dkv_finalize; rows past S are written too (the
        // buffer is padded to whole tiles) and never read
        const int slot = SCHED == SCHED_TABLE ? t.g : part;  // the run's head in a table
        const long long prow = ((long long)(b * p.Hkv + hk) * p.parts + slot) * p.NT + i * T + key_local;
        float* const pk = p.dkv_part + prow * D;
        float* const pv = p.dkv_part + (long long)p.B * p.Hkv * p.parts * p.NT * D + prow * D;
#pragma unroll
        for (int md = 0; md < C::DB; ++md) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 xk = {dK[md][4 * q4], dK[md][4 * q4 + 1], dK[md][4 * q4 + 2], dK[md][4 * q4 + 3]};
            const f32x4 xv = {dV[md][4 * q4], dV[md][4 * q4 + 1], dV[md][4 * q4 + 2], dV[md][4 * q4 + 3]};
            const int d0 = 32 * md + 8 * q4 + 4 * hg;
            *reinterpret_cast<f32x4*>(pk + d0) = xk;
            *reinterpret_cast<f32x4*>(pv + d0) = xv;
          }
        }
      } else if (t.seg_end) {
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

// Atomic reference only: dQ partial sums -> bf16 dq.  One thread per float of
// the accumulator, laid out as [tile][pass][wave slice][e][lane] with element
// e of lane l of wave w = row 32(w >> 2) + 16(e/4) + 4(l/16) + e%4 of the
// pass, feature 16(w & 3) + l%16.
__global__ __launch_bounds__(256) void bwd_finalize_wide64(FinParams p) {
  using C = Wide64Cfg;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)p.B * p.Hq * p.N * C::NP * C::NW * C::SLICE;
  if (idx >= total) return;
  if (__hip_atomic_load(p.ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  const int lane = (int)(idx % 64);
  long long rest = idx / 64;
  const int e = (int)(rest % 8);
  rest /= 8;
  const int w = (int)(rest % C::NW);
  rest /= C::NW;
  const int hp = (int)(rest % C::NP);
  rest /= C::NP;
  const int j = (int)(rest % p.N);
  const long long bh = rest / p.N;
  const int b = (int)(bh / p.Hq), h = (int)(bh % p.Hq);
  const int ql = hp * C::BQ + 32 * (w >> 2) + 16 * (e >> 2) + 4 * (lane >> 4) + (e & 3);
  const int row = j * C::T + ql;
  if (row < p.S)
    ((bf16*)p.dq)[((size_t)((size_t)b * p.S + row) * p.Hq + h) * C::D + 16 * (w & 3) + (lane & 15)] =
        (bf16)(p.dqacc[idx] * p.scale);
}

// ---------------------------------------------------------------------------
// Launch helpers

template <bool CAUSAL>
static int wide64_blocks_per_cu_impl() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, bwd_main_wide64<CAUSAL, SCHED_SHIFT>, 512, 0) != hipSuccess)
    return 0;
  return nb;
}

int bwd_wide64_blocks_per_cu(bool causal) {
  return causal ? wide64_blocks_per_cu_impl<true>() : wide64_blocks_per_cu_impl<false>();
}

template <bool CAUSAL>
static hipError_t launch_wide64_sched(int sched, const BwdParams& p, int grid, hipStream_t s) {
  switch (sched) {
    case SCHED_NAIVE:
      hipLaunchKernelGGL((bwd_main_wide64<CAUSAL, SCHED_NAIVE>), dim3(grid), dim3(512), 0, s, p);
      break;
    case SCHED_DESC:
      hipLaunchKernelGGL((bwd_main_wide64<CAUSAL, SCHED_DESC>), dim3(grid), dim3(512), 0, s, p);
      break;
    case SCHED_SHIFT:
      hipLaunchKernelGGL((bwd_main_wide64<CAUSAL, SCHED_SHIFT>), dim3(grid), dim3(512), 0, s, p);
      break;
    case SCHED_SYM:
      if constexpr (CAUSAL) {
        hipLaunchKernelGGL((bwd_main_wide64<CAUSAL, SCHED_SYM>), dim3(grid), dim3(512), 0, s, p);
        break;
      }
      return hipErrorInvalidValue;
    case SCHED_ATOMIC:
      hipLaunchKernelGGL((bwd_main_wide64<CAUSAL, SCHED_ATOMIC>), dim3(grid), dim3(512), 0, s, p);
      break;
    case SCHED_TABLE:
      hipLaunchKernelGGL((bwd_main_wide64<CAUSAL, SCHED_TABLE>), dim3(grid), dim3(512), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_wide64(bool causal, const BwdParams& p, int grid, hipStream_t s) {
  return causal ? launch_wide64_sched<true>(p.schedule, p, grid, s)
                : launch_wide64_sched<false>(p.schedule, p, grid, s);
}

hipError_t launch_finalize_wide64(const FinParams& p, hipStream_t s) {
  const long long total = (long long)p.B * p.Hq * p.N * Wide64Cfg::T * Wide64Cfg::D;
  const long long blocks = (total + 255) / 256;
  if (blocks < 1) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_finalize_wide64, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dash
