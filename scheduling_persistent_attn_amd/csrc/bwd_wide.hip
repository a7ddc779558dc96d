// Deterministic attention backward for gfx950, head dim 128, 256-key tiles.
//
// The same method and hand-off protocol as bwd_main (bwd.hip), with a
// key/value tile of 256 keys per unit instead of 128.  Per task of one unit
// the partial-sum traffic and the Q/dO re-reads are 12 T D bytes for 10 T^2 D
// FLOPs, so doubling the keys a unit holds halves the bytes moved per FLOP
// (about 105 -> 210 FLOP per byte at D = 128).  A unit's dK/dV for 256 keys
// are 256 KiB of fp32, half of a compute unit's registers, so the workgroup
// has eight waves (two per SIMD, 256 registers each): wave w owns keys
// [32w, 32w+32) and keeps their dK/dV (128 registers) and V rows (the B
// operand of dP, 32 registers) for the whole run of the tile, all in vector
// registers.  The K tile sits
// in LDS, where it serves as the B operand of S (each wave's own rows) and,
// through transposing reads, as the B operand of dQ = dS K.  Two waves per
// SIMD let one wave's softmax, LDS and memory work run beside the other's
// matrix products.
//
// Per pass of 32 query rows each wave computes, for its 32 keys,
//   S - lse/scale = Q K^T, dP - Dl = dO V^T, P, dS  (v_mfma_f32_32x32x16_bf16)
//   dV^T += dO^T P, dK^T += Q^T dS                  (v_mfma_f32_32x32x16_bf16)
// writes dS to LDS, and forms its 32-row x 16-feature slice of the dQ of the
// pass two passes back, dQ = dS K over all 256 keys
// (v_mfma_f32_16x16x32_bf16), followed by the ordered reduction of that slice
// (the turn counters of bwd_common.h; one counter per slice).
//
// Accumulator layouts.  32x32x16: register r of lane l holds column l % 32 and
// row 8(r/4) + 4(l/32) + r%4.  16x16x32: register r of lane l holds column
// l % 16 and row 4(l/16) + r; its A operand (16 rows x 32 k) is row l % 16,
// k 8(l/16) .. +7 of lane l, its B operand (32 k x 16 columns) column l % 16,
// k 8(l/16) .. +7.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwd_common.h"
#include "kernels.h"
#include "lds_layout.h"
#include "schedule.h"

namespace dash {

struct WideCfg {
  static constexpr int D = 128, T = 256;
  static constexpr int NW = 8;          // waves; wave w owns keys [32w, 32w+32)
  static constexpr int DB = D / 32;     // 32-wide feature blocks of dK/dV
  static constexpr int BQ = 32;         // query rows per pass
  static constexpr int NP = T / BQ;     // passes per task
  static constexpr int KBD = D / 16;    // 16-wide k-blocks over the head dim
  static constexpr int KBK = T / 32;    // 32-key k-steps of the dQ product
  static constexpr int FQ = D / NW;     // dQ features per wave
  static constexpr int SLICE = BQ * FQ; // floats per dQ slice
  static constexpr int RBD = 2 * D;     // bytes per row of a Q/dO/K tile
  static constexpr int RBS = 2 * T;     // bytes per row of the dS block
  static constexpr int K_TILE = T * RBD, Q_TILE = BQ * RBD, S_TILE = BQ * RBS;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_Q = K_TILE;                // + buf * Q_TILE
  static constexpr int OFF_DO = OFF_Q + 2 * Q_TILE;   // + buf * Q_TILE
  static constexpr int OFF_DS = OFF_DO + 2 * Q_TILE;  // + buf * S_TILE, 3 buffers
  static constexpr int OFF_LD = OFF_DS + 3 * S_TILE;  // [buf][-lse/scale | -Dl][BQ] fp32
  static constexpr int OFF_MISC = OFF_LD + 2 * 2 * 4 * BQ;
  static constexpr int LDS_BYTES = OFF_MISC + 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(FQ == 16 && SLICE == 512, "one 32 x 16 dQ slice per wave and pass");
};

// Per-lane LDS byte offsets of the wide kernel (see LaneOffs in bwd.hip for
// the idea: every access pattern is a per-lane base XOR or plus a constant).
struct WideOffs {
  int a;      // 16-byte row reads of Q/dO/K: row c, chunk 2kb + hg is a ^ 32kb
  int tq[2];  // transposing reads of Q/dO rows 8h8 + 4hg + (s16 >> 2), feature
              // block md: tq[h8] ^ 64md
  int kt[2];  // transposing reads of K rows 8g16 + 4h + (s16 >> 2), features
              // 16w .. 16w+15 (+32 rows per k-step: + 8192 kb)
  int sA;     // dQ A operand: dS row s16, keys 32kb + 8g16 .. : sA ^ (kb << 6)
              // (+16 rows: + 8192)
  int wr;     // dS element writes of row 8(x >> 2) + 4hg + (x & 3), key 32w + c:
              // (wr ^ wx(x)) + wy(x)
  __device__ __forceinline__ int A(int kb) const { return a ^ (32 * kb); }
  __device__ __forceinline__ int Tq(int md, int h8) const { return tq[h8] ^ (64 * md); }
  __device__ __forceinline__ int SA(int kb, int rb) const { return (sA ^ (kb << 6)) + rb * 8192; }
  static constexpr int wx(int x) { return ((8 * ((x >> 2) & 1)) | (x & 3)) << 4; }
  static constexpr int wy(int x) { return (8 * (x >> 2) + (x & 3)) * 512; }
  __device__ __forceinline__ int W(int x) const { return (wr ^ wx(x)) + wy(x); }
};

// dQ slice of one pass: rows 0..31 of the pass x features 16w .. 16w+15, over
// the 256 keys of the tile; A = dS rows (LDS), B = K^T (transposing reads of
// the K tile), accumulated onto c (the loaded partial sum, or zeros).
__device__ __forceinline__ DQ2 wide_dq_products(const char* lS, const char* lK, const WideOffs& o, DQ2 c) {
  using C = WideCfg;
  bf16x8 fa0[2], fa1[2], fb[2];
  fa0[0] = lds_read16(lS, o.SA(0, 0));
  fa1[0] = lds_read16(lS, o.SA(0, 1));
  fb[0] = lds_read_tr(lK, o.kt[0], o.kt[1]);
#pragma unroll
  for (int kb = 0; kb < C::KBK; ++kb) {
    if (kb + 1 < C::KBK) {
      fa0[(kb + 1) & 1] = lds_read16(lS, o.SA(kb + 1, 0));
      fa1[(kb + 1) & 1] = lds_read16(lS, o.SA(kb + 1, 1));
      fb[(kb + 1) & 1] = lds_read_tr(lK, o.kt[0] + (kb + 1) * 8192, o.kt[1] + (kb + 1) * 8192);
    }
    c.v[0] = mfma16(fa0[kb & 1], fb[kb & 1], c.v[0]);
    c.v[1] = mfma16(fa1[kb & 1], fb[kb & 1], c.v[1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  return c;
}

// P = exp2((S - lse/scale) * scale * log2e), dS = P * (dP - Dl), rounded to
// bf16 as the B operands of dV and dK.
__device__ __forceinline__ void wide_softmax(const f32x16& sacc, const f32x16& dpacc, float scale_log2e,
                                             bf16x8* pb, bf16x8* dsb) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float pv = __builtin_amdgcn_exp2f(sacc[r] * scale_log2e);
    pb[r >> 3][r & 7] = (bf16)pv;
    dsb[r >> 3][r & 7] = (bf16)(pv * dpacc[r]);
  }
}

// dV^T += dO^T P and dK^T += Q^T dS over the 32 query rows of the pass,
// fragments one step ahead, with the dS element writes to lS spread over the
// steps.
__device__ __forceinline__ void wide_dvdk(const char* lQ, const char* lO, const WideOffs& o, const bf16x8* pb,
                                          const bf16x8* dsb, f32x16* dK, f32x16* dV, char* lS) {
  using C = WideCfg;
  constexpr int X = 2 * C::DB;  // product steps
  constexpr int WPS = 16 / X;   // dS element writes per step
  bf16x8 fa[2], fb[2];
  fa[0] = lds_read_tr(lO, o.Tq(0, 0), o.Tq(0, 1));
  fb[0] = lds_read_tr(lQ, o.Tq(0, 0), o.Tq(0, 1));
#pragma unroll
  for (int x = 0; x < X; ++x) {
    const int md = x >> 1, kq = x & 1;
    if (x + 1 < X) {
      const int md2 = (x + 1) >> 1, kq2 = (x + 1) & 1;
      const int base = 16 * kq2 * C::RBD;
      fa[(x + 1) & 1] = lds_read_tr(lO, o.Tq(md2, 0) + base, o.Tq(md2, 1) + base);
      fb[(x + 1) & 1] = lds_read_tr(lQ, o.Tq(md2, 0) + base, o.Tq(md2, 1) + base);
    }
    dV[md] = mfma(fa[x & 1], pb[kq], dV[md]);
    dK[md] = mfma(fb[x & 1], dsb[kq], dK[md]);
#pragma unroll
    for (int e = 0; e < WPS; ++e) {
      const int r = x * WPS + e;
      lds_write_bf16(lS + o.W(r & 7) + (r >> 3) * 16 * C::RBS, dsb[r >> 3], r & 7);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pass of the current task plus two stages of the ordered reductions of
// earlier passes, as pass_body in bwd.hip: the dQ slice `ld` (two passes
// back) is formed on its loaded partial sum and stored; the turn of `prev`
// (polled at the pass start) is taken and its partial sum loaded; slice `rel`
// (stored at the end of the previous pass) is published after the S/dP
// products.
template <bool CAUSAL, bool ATOMIC>
__device__ __forceinline__ void wide_pass(const char* lQ, const char* lO, const char* lL, const char* lK,
                                          char* lS_cur, const char* lS_ld, const WideOffs& o, int lane, int w,
                                          float scale_log2e, bool masked, unsigned zb, const bf16x8* vB,
                                          f32x16* dK, f32x16* dV, const WideSlice& ld, bool ld_on, DQ2& dq_ld,
                                          const WideSlice& prev, const WideSlice& rel, bool rel_on,
                                          const int* poll_ptr, int poll_expect, int polled, int acc_bytes,
                                          const BwdParams& p, int rs, bf16* gdq, unsigned dq_bytes,
                                          const PassStage<128, 32, 8>* stage, bool stage_on, char* st_q,
                                          char* st_o, char* st_l) {
  using C = WideCfg;
  const int hg = lane >> 5;
  // ---- S and dP; the accumulators start at -lse/scale and -Dl of their rows
  f32x16 sa, pa;
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    const f32x4 l = *reinterpret_cast<const f32x4*>(lL + 4 * (8 * k4 + 4 * hg));
    const f32x4 d = *reinterpret_cast<const f32x4*>(lL + 4 * C::BQ + 4 * (8 * k4 + 4 * hg));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sa[4 * k4 + e] = l[e];
      pa[4 * k4 + e] = d[e];
    }
  }
  if (masked) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = ((zb >> r) & 1u) ? -__builtin_inff() : sa[r];
  }
  {
    const int kown = 32 * w * C::RBD;  // this wave's K rows
    bf16x8 fq[2], fd[2], fk[2];
    fq[0] = lds_read16(lQ, o.A(0));
    fd[0] = lds_read16(lO, o.A(0));
    fk[0] = lds_read16(lK, o.A(0) + kown);
#pragma unroll
    for (int kb = 0; kb < C::KBD; ++kb) {
      if (kb + 1 < C::KBD) {
        fq[(kb + 1) & 1] = lds_read16(lQ, o.A(kb + 1));
        fd[(kb + 1) & 1] = lds_read16(lO, o.A(kb + 1));
        fk[(kb + 1) & 1] = lds_read16(lK, o.A(kb + 1) + kown);
      }
      sa = mfma(fq[kb & 1], fk[kb & 1], sa);
      pa = mfma(fd[kb & 1], vB[kb], pa);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- publish slice `rel`, whose partial-sum stores ended the previous
  // pass.  Since then this wave issued exactly: the two partial-sum loads of
  // `prev` (wide_acc_load, always two b128 loads, out of range when nothing
  // is added), the next pass's staging loads (stage_load: 2 * KQ = 2 tile
  // loads and one per-row value load, all unconditional) and one turn poll,
  // i.e. 2 + 3 + 1 = 6 vector-memory operations.  They retire in issue order,
  // so once at most 6 are outstanding the stores have completed.
  if constexpr (!ATOMIC) {
    static_assert(PassStage<128, 32, 8>::KQ == 1, "counted wait below");
    if (rel_on) {
      order_point();
      wait_vm<6>();
      order_point();
      release(rel, lane);
    }
  }

  // ---- softmax, then dV^T += dO^T P, dK^T += Q^T dS; dS -> LDS
  bf16x8 pb[2], dsb[2];
  wide_softmax(sa, pa, scale_log2e, pb, dsb);
  // the dS element writes take the bf16 halves of these registers as they
  // are, instead of converting every element once more
  asm volatile("" : "+v"(dsb[0]), "+v"(dsb[1]));
  wide_dvdk(lQ, lO, o, pb, dsb, dK, dV, lS_cur);

  // ---- dQ of the slice two passes back on its loaded partial sum
  __builtin_amdgcn_sched_barrier(0);
  const DQ2 dq = wide_dq_products(lS_ld, lK, o, dq_ld);

  // ---- the next pass's inputs into the other LDS buffer
  if (stage_on) stage_store<128, 32, 8>(*stage, st_q, st_o, st_l, w, lane);

  // ---- turn of the previous slice, the stores of the slice two passes back,
  // then the previous slice's partial sum (the last vector memory operations
  // of the pass)
  order_point();
  if constexpr (!ATOMIC) acquire(poll_ptr, poll_expect, polled, p.ctrl, p.spin_ticks, lane);
  order_point();
  if (ld_on) wide_acc_finish<ATOMIC>(ld, dq, lane, rs, p.scale, gdq, dq_bytes);
  order_point();
  if constexpr (ATOMIC) {
    dq_ld.v[0] = f32x4{};
    dq_ld.v[1] = f32x4{};
  } else {
    dq_ld = wide_acc_load(prev.acc, acc_bytes, lane);
  }
  order_point();
}

template <bool CAUSAL, int SCHED>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512)))
__attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_main_wide(BwdParams p) {
  using C = WideCfg;
  constexpr int T = C::T, D = C::D, BQ = C::BQ, NP = C::NP;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const char* const lK = smem + C::OFF_K;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & (C::NW - 1);
  const int lane = tid & 63, c = lane & 31, hg = lane >> 5, g16 = lane >> 4, s16 = lane & 15;
  constexpr int mask = CAUSAL ? MASK_CAUSAL : MASK_FULL;
  constexpr bool atomic_dq = SCHED == SCHED_ATOMIC;
  const int N = p.N, G = p.G, S = p.S;
  const int rsq = p.Hq * D;  // row stride of q / dout / dq
  bf16* const gdq = (bf16*)p.dq;
  // bytes of dq (below 2^32: the host keeps element offsets below 2^31)
  const unsigned dq_bytes = (unsigned)p.B * (unsigned)S * (unsigned)p.Hq * (unsigned)(2 * D);

  // ---- per-lane LDS offsets
  WideOffs o;
  o.a = lds_phys<C::RBD>(c, hg);
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8) {
    const int col = 16 * (g16 & 1) + 4 * (s16 & 3);
    o.tq[h8] = lds_phys<C::RBD>(8 * h8 + 4 * hg + (s16 >> 2), col >> 3) + 2 * (col & 7);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = 16 * w + 4 * (s16 & 3);
    o.kt[h] = lds_phys<C::RBD>(8 * g16 + 4 * h + (s16 >> 2), col >> 3) + 2 * (col & 7);
  }
  o.sA = ds_phys(s16, g16);
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
  WideSlice prev = {}, ld = {}, rel = {};
  bool have_prev = false, have_ld = false, rel_pending = false;
  DQ2 dq_ld = {};
  int sb = 0;
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
      const int r00 = j * T;
      const int dq_off0 = (b * S + r00) * rsq + h * D + 16 * w + s16;

      for (int hp = 0; hp < NP; ++hp, ++gp) {
        const int buf = gp & 1;
        const char* const lQ = smem + C::OFF_Q + buf * C::Q_TILE;
        const char* const lO = smem + C::OFF_DO + buf * C::Q_TILE;
        const char* const lL = smem + C::OFF_LD + buf * 2 * 4 * BQ;
        char* const lS_cur = smem + C::OFF_DS + sb * C::S_TILE;
        const int sb_ld = sb == 0 ? 1 : (sb == 1 ? 2 : 0);  // two passes back
        const char* const lS_ld = smem + C::OFF_DS + sb_ld * C::S_TILE;
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

        const bool need_turn = !atomic_dq && have_prev && prev.rank > 0;
        const int* const poll_ptr = need_turn ? prev.cnt : p.ctrl + 3;
        const int poll_expect = need_turn ? prev.rank : 0;
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

        unsigned zb = 0;
        if (CAUSAL && i == j) zb = w > hp ? 0xffffu : (w == hp ? diag_bits : 0u);
        if (kv_tail && !key_ok) zb = 0xffffu;
        wide_pass<CAUSAL, atomic_dq>(lQ, lO, lL, lK, lS_cur, lS_ld, o, lane, w, p.scale_log2e, masked, zb, vB, dK,
                                     dV, ld, have_ld, dq_ld, prev, rel, rel_pending, poll_ptr, poll_expect, polled,
                                     acc_bytes, p, rsq, gdq, dq_bytes, &stage, stage_next,
                                     smem + C::OFF_Q + (buf ^ 1) * C::Q_TILE,
                                     smem + C::OFF_DO + (buf ^ 1) * C::Q_TILE,
                                     smem + C::OFF_LD + (buf ^ 1) * 2 * 4 * BQ);
        acc_tail = true;
        rel_pending = false;  // published inside the pass body
        if (have_ld && !atomic_dq) {
          rel = ld;
          rel_pending = true;
        }
        ld = prev;
        have_ld = have_prev;

        if (hp == NP - 1 && t.seg_end) {
          // last pass of this KV tile's run: finish the two open slices while
          // the K tile is still in LDS
          __syncthreads();  // every wave's dS of this pass is in LDS
          const int sb_prev = sb == 0 ? 2 : sb - 1;
          if (have_ld) {
            const DQ2 dq = wide_dq_products(smem + C::OFF_DS + sb_prev * C::S_TILE, lK, o, dq_ld);
            wide_acc_finish<atomic_dq>(ld, dq, lane, rsq, p.scale, gdq, dq_bytes);
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
          const DQ2 dq = wide_dq_products(lS_cur, lK, o, wide_acc_load(cur.acc, ct ? 2048 : 0, lane));
          wide_acc_finish<atomic_dq>(cur, dq, lane, rsq, p.scale, gdq, dq_bytes);
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
// e of lane l = row 16(e/4) + 4(l/16) + e%4, feature 16w + l%16 of the pass.
__global__ __launch_bounds__(256) void bwd_finalize_wide(FinParams p) {
  using C = WideCfg;
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
  const int ql = hp * C::BQ + 16 * (e >> 2) + 4 * (lane >> 4) + (e & 3);
  const int row = j * C::T + ql;
  if (row < p.S)
    ((bf16*)p.dq)[((size_t)((size_t)b * p.S + row) * p.Hq + h) * C::D + 16 * w + (lane & 15)] =
        (bf16)(p.dqacc[idx] * p.scale);
}

// dK/dV of split groups: dk[b, s, hk, :] = scale * sum over the parts of
// their fp32 partials, added in ascending part order (a fixed order, so the
// result is reproducible), then rounded to bf16; dv likewise without the
// scale.  The parts are query-head parts of a closed-form schedule, or the
// single heads of a per-head task table.  One thread per four features.
__global__ __launch_bounds__(256) void bwd_dkv_finalize(DkvFinParams p) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int q4n = p.D / 4;
  const long long total = 2LL * p.B * p.Hkv * p.S * q4n;
  if (idx >= total) return;
  if (__hip_atomic_load(p.ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  // after a table run: only if that table wrote per-head partials
  if (p.need_mark && __hip_atomic_load(p.ctrl + 6, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) return;
  const int q4 = (int)(idx % q4n);
  long long rest = idx / q4n;
  const int hk = (int)(rest % p.Hkv);
  rest /= p.Hkv;
  const int s = (int)(rest % p.S);
  rest /= p.S;
  const int b = (int)(rest % p.B);
  const int which = (int)(rest / p.B);  // 0: dK, 1: dV
  const long long half = (long long)p.B * p.Hkv * p.parts * p.NT * p.D;
  const float* src = p.dkv_part + which * half + (((long long)(b * p.Hkv + hk) * p.parts) * p.NT + s) * p.D + 4 * q4;
  f32x4 acc = *reinterpret_cast<const f32x4*>(src);
  for (int k = 1; k < p.parts; ++k) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(src + (long long)k * p.NT * p.D);
    acc[0] += x[0];
    acc[1] += x[1];
    acc[2] += x[2];
    acc[3] += x[3];
  }
  const float sc = which == 0 ? p.scale : 1.0f;
  bf16x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (bf16)(acc[e] * sc);
  bf16* const dst = (bf16*)(which == 0 ? p.dk : p.dv);
  *reinterpret_cast<bf16x4*>(dst + (((long long)b * p.S + s) * p.Hkv + hk) * p.D + 4 * q4) = o;
}

// ---------------------------------------------------------------------------
// Launch helpers

template <bool CAUSAL>
static int wide_blocks_per_cu_impl() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, bwd_main_wide<CAUSAL, SCHED_SHIFT>, 512, 0) != hipSuccess)
    return 0;
  return nb;
}

int bwd_wide_blocks_per_cu(bool causal) {
  return causal ? wide_blocks_per_cu_impl<true>() : wide_blocks_per_cu_impl<false>();
}

template <bool CAUSAL>
static hipError_t launch_wide_sched(int sched, const BwdParams& p, int grid, hipStream_t s) {
  switch (sched) {
    case SCHED_NAIVE:
      hipLaunchKernelGGL((bwd_main_wide<CAUSAL, SCHED_NAIVE>), dim3(grid), dim3(512), 0, s, p);
      break;
    case SCHED_DESC:
      hipLaunchKernelGGL((bwd_main_wide<CAUSAL, SCHED_DESC>), dim3(grid), dim3(512), 0, s, p);
      break;
    case SCHED_SHIFT:
      hipLaunchKernelGGL((bwd_main_wide<CAUSAL, SCHED_SHIFT>), dim3(grid), dim3(512), 0, s, p);
      break;
    case SCHED_SYM:
      if constexpr (CAUSAL) {
        hipLaunchKernelGGL((bwd_main_wide<CAUSAL, SCHED_SYM>), dim3(grid), dim3(512), 0, s, p);
        break;
      }
      return hipErrorInvalidValue;
    case SCHED_ATOMIC:
      hipLaunchKernelGGL((bwd_main_wide<CAUSAL, SCHED_ATOMIC>), dim3(grid), dim3(512), 0, s, p);
      break;
    case SCHED_TABLE:
      hipLaunchKernelGGL((bwd_main_wide<CAUSAL, SCHED_TABLE>), dim3(grid), dim3(512), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_wide(bool causal, const BwdParams& p, int grid, hipStream_t s) {
  return causal ? launch_wide_sched<true>(p.schedule, p, grid, s) : launch_wide_sched<false>(p.schedule, p, grid, s);
}

hipError_t launch_dkv_finalize(const DkvFinParams& p, hipStream_t s) {
  const long long total = 2LL * p.B * p.Hkv * p.S * (p.D / 4);
  const long long blocks = (total + 255) / 256;
  if (blocks < 1) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dkv_finalize, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_finalize_wide(const FinParams& p, hipStream_t s) {
  const long long total = (long long)p.B * p.Hq * p.N * WideCfg::T * WideCfg::D;
  const long long blocks = (total + 255) / 256;
  if (blocks < 1) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_finalize_wide, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dash
