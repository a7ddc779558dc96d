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
// LDS tile layouts.
//
// Row-major tile with CH 16-byte chunks per row: chunk u of row r is stored at
// chunk (u ^ (r & (min(CH,16) - 1))), so that the 32 rows a wave reads at one
// column fall into distinct banks.
template <int CH>
__device__ __forceinline__ int rm_off(int row, int chunk) {  // element offset
  constexpr int M = (CH < 16 ? CH : 16) - 1;
  return (row * CH + (chunk ^ (row & M))) * 8;
}
// Transposed tile: row d holds the T values of one feature, in 8-byte chunks
// of 4 consecutive sequence positions; chunk v of row d is stored at
// v ^ ((d & 15) ^ ((d >> 3) & 15)), which keeps both the reads (16
// consecutive rows, one chunk) and the writes (rows 8 apart, one chunk)
// free of bank conflicts.
template <int C8>
__device__ __forceinline__ int tr_off(int d, int v) {
  const int sw = ((d & 15) ^ ((d >> 3) & 15)) & (C8 - 1);
  return (d * C8 + (v ^ sw)) * 4;
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

// ---------------------------------------------------------------------------
template <int D, int T, bool CAUSAL>
struct BwdCfg {
  static constexpr int NW = T / 32;       // waves
  static constexpr int NT = 64 * NW;      // threads
  static constexpr int KBD = D / 16;      // k-blocks over the head dim
  static constexpr int KBT = T / 16;      // k-blocks over a tile
  static constexpr int DB = D / 32;       // 32-wide feature blocks
  static constexpr int QB = T / 32;       // 32-row blocks of a tile
  static constexpr int MQ = DB;           // dQ row blocks per wave
  static constexpr int UPT = D / 64;      // 4x8 load units per thread per tile
  static constexpr int CHD = D / 8;       // 16-byte chunks per Q/dO row
  static constexpr int CHT = T / 8;       // 16-byte chunks per dS row
  static constexpr int C8 = T / 4;        // 8-byte chunks per transposed row
  static constexpr int LDS_ELEMS = 4 * T * D + T * T;
  static_assert(T >= D, "tile must be at least the head dim");
  static_assert(UPT >= 1, "head dim must be a multiple of 64");
};

template <int D, int T, bool CAUSAL, int SCHED>
__global__ __attribute__((amdgpu_flat_work_group_size(2 * T, 2 * T)))
__attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_main(BwdParams p) {
  using C = BwdCfg<D, T, CAUSAL>;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::LDS_ELEMS];
  bf16* const sQ = smem;
  bf16* const sQT = sQ + T * D;
  bf16* const sdO = sQT + D * T;
  bf16* const sdOT = sdO + T * D;
  bf16* const sdS = sdOT + D * T;

  // Lane-derived values are refreshed behind an opaque move at every task so
  // that the many swizzled LDS offsets built from them are recomputed inside
  // the task instead of being hoisted (and spilled) across the whole loop.
  int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lane = tid & 63, c = lane & 31, hg = lane >> 5;
  const int qg = w / C::DB, db = w % C::DB;  // this wave's dQ block
  const int mask = CAUSAL ? MASK_CAUSAL : MASK_FULL;
  const int N = p.N, G = p.G, S = p.S;
  constexpr bool atomic_dq = SCHED == SCHED_ATOMIC;
  const bf16* const gq = (const bf16*)p.q;
  const bf16* const gk = (const bf16*)p.k;
  const bf16* const gv = (const bf16*)p.v;
  const bf16* const gdo = (const bf16*)p.dout;

  bf16x8 kB[C::KBD], vB[C::KBD], ktB[C::KBT];
  f32x16 dK[C::DB], dV[C::DB];
  bf16x8 rq[C::UPT][4], rdo[C::UPT][4];

  // global -> registers: the Q and dO rows of query tile j of head h
  // global -> registers: the Q and dO rows of query tile j of head h.
  // Element offsets fit in 32 bits (checked on the host).  Rows past S
  // (a partial last tile) read a valid row and are replaced by zeros.
  auto load_qdo = [&](int b, int h, int j) {
    const int rs = p.Hq * D;
    const int base = (b * S + j * T) * rs + h * D;
    const bool full = (j + 1) * T <= S;
    const int last_row = S - 1 - j * T;
#pragma unroll
    for (int u = 0; u < C::UPT; ++u) {
      const int un = tid + u * C::NT;
      const int cu = un % C::CHD, rg = un / C::CHD;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = 4 * rg + e;
        const int rc = full ? rl : min(rl, last_row);
        const int off = base + rc * rs + 8 * cu;
        rq[u][e] = *reinterpret_cast<const bf16x8*>(gq + off);
        rdo[u][e] = *reinterpret_cast<const bf16x8*>(gdo + off);
      }
    }
    if (!full) {
#pragma unroll
      for (int u = 0; u < C::UPT; ++u) {
        const int un = tid + u * C::NT;
        const int rg = un / C::CHD;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (4 * rg + e > last_row) {
            rq[u][e] = zero8();
            rdo[u][e] = zero8();
          }
        }
      }
    }
  };
  // registers -> LDS, row-major and transposed copies
  auto store_qdo = [&]() {
#pragma unroll
    for (int u = 0; u < C::UPT; ++u) {
      const int un = tid + u * C::NT;
      const int cu = un % C::CHD, rg = un / C::CHD;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<bf16x8*>(sQ + rm_off<C::CHD>(4 * rg + e, cu)) = rq[u][e];
        *reinterpret_cast<bf16x8*>(sdO + rm_off<C::CHD>(4 * rg + e, cu)) = rdo[u][e];
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int d = 8 * cu + x;
        bf16x4 tq, tdo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tq[e] = rq[u][e][x];
          tdo[e] = rdo[u][e][x];
        }
        *reinterpret_cast<bf16x4*>(sQT + tr_off<C::C8>(d, rg)) = tq;
        *reinterpret_cast<bf16x4*>(sdOT + tr_off<C::C8>(d, rg)) = tdo;
      }
    }
  };
  // A fragment (m = feature row, k = 16 sequence positions in the permuted
  // accumulator order) from a transposed tile
  auto read_tr = [&](const bf16* base, int d, int q0) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(base + tr_off<C::C8>(d, q0 >> 2));
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(base + tr_off<C::C8>(d, (q0 >> 2) + 2));
    bf16x8 a;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[s] = lo[s];
      a[s + 4] = hi[s];
    }
    return a;
  };

  for (;;) {
    __syncthreads();
    if (tid == 0) {
      int it = atomicAdd(p.ctrl, 1);
      if (__hip_atomic_load(p.ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
        it = p.total_items;
      reinterpret_cast<int*>(sdS)[0] = it;
    }
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(sdS)[0]);
    if (item >= p.total_items) break;
    const int grp = item / p.items_per_group;
    const int local = item - grp * p.items_per_group;
    const int b = grp / p.Hkv, hk = grp - b * p.Hkv;
    const int len = item_len(mask, SCHED, N, G, local);

    {
      const Task t0 = task_at(mask, SCHED, N, G, local, 0);
      load_qdo(b, hk * G + t0.g, t0.j);
    }
    __syncthreads();  // everyone has read the item index held in sdS
    store_qdo();

    for (int step = 0; step < len; ++step) {
      asm volatile("" : "+v"(tid));
      lane = tid & 63;
      c = lane & 31;
      hg = lane >> 5;
      const Task t = task_at(mask, SCHED, N, G, local, step);
      const int i = t.i, j = t.j, h = hk * G + t.g;
      if (t.seg_begin) {
        // K/V fragments of this wave's 32 keys; K^T fragments of its dQ slice
        const int rs = p.Hkv * D;
        const int base = (b * S + i * T) * rs + hk * D;
        const int last_key = S - 1 - i * T;
        const bool full = (i + 1) * T <= S;
        {
          const int kl = 32 * w + c;
          const int off = base + (full ? kl : min(kl, last_key)) * rs + 8 * hg;
#pragma unroll
          for (int kb = 0; kb < C::KBD; ++kb) {
            kB[kb] = *reinterpret_cast<const bf16x8*>(gk + off + 16 * kb);
            vB[kb] = *reinterpret_cast<const bf16x8*>(gv + off + 16 * kb);
          }
          if (!full && kl > last_key) {
#pragma unroll
            for (int kb = 0; kb < C::KBD; ++kb) {
              kB[kb] = zero8();
              vB[kb] = zero8();
            }
          }
        }
        {
          const int off = base + 32 * db + c;
#pragma unroll
          for (int kb = 0; kb < C::KBT; ++kb) {
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) {
              const int kl = 16 * kb + 8 * hg + s8;
              const int kc = full ? kl : min(kl, last_key);
              const bf16 x = gk[off + kc * rs];
              ktB[kb][s8] = (full || kl <= last_key) ? x : (bf16)0.0f;
            }
          }
        }
#pragma unroll
        for (int md = 0; md < C::DB; ++md) {
          dK[md] = f32x16{};
          dV[md] = f32x16{};
        }
      }
      __syncthreads();  // Q/dO of this task are in LDS; sdS is free

      const bool has_next = step + 1 < len;

      const int rowbase = ((b * p.Hq + h) * N + j) * T;
      const bool diag = CAUSAL && i == j;
      const bool kv_tail = (i + 1) * T > S;
      const int key_local = 32 * w + c;
      const bool key_ok = i * T + key_local < S;

#pragma unroll 1
      for (int mt = 0; mt < C::QB; ++mt) {
        if (diag && w > mt) {
          // keys of this wave are all after these queries: dS block is zero
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = 32 * mt + 8 * (r >> 2) + 4 * hg + (r & 3);
            sdS[rm_off<C::CHT>(ql, key_local >> 3) + (key_local & 7)] = (bf16)0.0f;
          }
          continue;
        }
        f32x16 sacc = {}, dpacc = {};
        {
          bf16x8 fq[2], fd[2];
          fq[0] = *reinterpret_cast<const bf16x8*>(sQ + rm_off<C::CHD>(32 * mt + c, hg));
          fd[0] = *reinterpret_cast<const bf16x8*>(sdO + rm_off<C::CHD>(32 * mt + c, hg));
#pragma unroll
          for (int kb = 0; kb < C::KBD; ++kb) {
            if (kb + 1 < C::KBD) {
              fq[(kb + 1) & 1] = *reinterpret_cast<const bf16x8*>(
                  sQ + rm_off<C::CHD>(32 * mt + c, 2 * (kb + 1) + hg));
              fd[(kb + 1) & 1] = *reinterpret_cast<const bf16x8*>(
                  sdO + rm_off<C::CHD>(32 * mt + c, 2 * (kb + 1) + hg));
            }
            sacc = mfma(fq[kb & 1], kB[kb], sacc);
            dpacc = mfma(fd[kb & 1], vB[kb], dpacc);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        f32x4 l2[4], dl[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          l2[k4] = *reinterpret_cast<const f32x4*>(p.lse2 + rowbase + 32 * mt + 8 * k4 + 4 * hg);
          dl[k4] = *reinterpret_cast<const f32x4*>(p.delta + rowbase + 32 * mt + 8 * k4 + 4 * hg);
        }
        bf16x8 pb[2], dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(sacc[r] * p.scale_log2e - l2[r >> 2][r & 3]);
          if (diag && mt == w) {
            const int ql = 32 * mt + 8 * (r >> 2) + 4 * hg + (r & 3);
            if (key_local > ql) pv = 0.0f;
          }
          if (kv_tail && !key_ok) pv = 0.0f;
          const float ds = pv * (dpacc[r] - dl[r >> 2][r & 3]);
          pb[r >> 3][r & 7] = (bf16)pv;
          dsb[r >> 3][r & 7] = (bf16)ds;
        }
        {
          // (md, kq) pairs in order; fragments for the next pair are read
          // while the current pair multiplies
          bf16x8 fv[2], fk[2];
          fv[0] = read_tr(sdOT, c, 32 * mt + 4 * hg);
          fk[0] = read_tr(sQT, c, 32 * mt + 4 * hg);
#pragma unroll
          for (int x = 0; x < 2 * C::DB; ++x) {
            const int md = x >> 1, kq = x & 1;
            if (x + 1 < 2 * C::DB) {
              const int md1 = (x + 1) >> 1, kq1 = (x + 1) & 1;
              fv[(x + 1) & 1] = read_tr(sdOT, 32 * md1 + c, 32 * mt + 16 * kq1 + 4 * hg);
              fk[(x + 1) & 1] = read_tr(sQT, 32 * md1 + c, 32 * mt + 16 * kq1 + 4 * hg);
            }
            dV[md] = mfma(fv[x & 1], pb[kq], dV[md]);
            dK[md] = mfma(fk[x & 1], dsb[kq], dK[md]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * mt + 8 * (r >> 2) + 4 * hg + (r & 3);
          sdS[rm_off<C::CHT>(ql, key_local >> 3) + (key_local & 7)] = dsb[r >> 3][r & 7];
        }
      }
      __syncthreads();  // all reads of this task's Q/dO done; dS complete
      // next task's Q/dO into LDS (the dQ product below reads only dS)
      if (has_next) {
        const Task tn = task_at(mask, SCHED, N, G, local, step + 1);
        load_qdo(b, hk * G + tn.g, tn.j);
        store_qdo();
      }

      // dQ slice of this wave: rows [32*MQ*qg, +32*MQ), features [32*db, +32)
      f32x16 dq[C::MQ];
#pragma unroll
      for (int m = 0; m < C::MQ; ++m) dq[m] = f32x16{};
      {
        // two k-blocks of dS fragments in flight: load kb+1, multiply kb
        bf16x8 fa[2][C::MQ];
#pragma unroll
        for (int m = 0; m < C::MQ; ++m)
          fa[0][m] = *reinterpret_cast<const bf16x8*>(
              sdS + rm_off<C::CHT>(32 * (qg * C::MQ + m) + c, hg));
#pragma unroll
        for (int kb = 0; kb < C::KBT; ++kb) {
          if (kb + 1 < C::KBT) {
#pragma unroll
            for (int m = 0; m < C::MQ; ++m)
              fa[(kb + 1) & 1][m] = *reinterpret_cast<const bf16x8*>(
                  sdS + rm_off<C::CHT>(32 * (qg * C::MQ + m) + c, 2 * (kb + 1) + hg));
          }
#pragma unroll
          for (int m = 0; m < C::MQ; ++m) dq[m] = mfma(fa[kb & 1][m], ktB[kb], dq[m]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ordered (or, for the reference, atomic) reduction into dQ
      const int tile = (b * p.Hq + h) * N + j;
      float* const acc = p.dqacc + (tile * C::NW + w) * (C::MQ * 1024);
      if constexpr (atomic_dq) {
        // element r of row block m of lane l at (m*16 + r)*64 + l: each
        // atomic instruction covers 64 consecutive floats
#pragma unroll
        for (int m = 0; m < C::MQ; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            unsafeAtomicAdd(acc + (m * 16 + r) * 64 + lane, dq[m][r]);
      } else {
        int* const cnt = p.counters + tile * C::NW + w;
        const int rank = t.rank;
        const bool last = rank == contributors(mask, N, j) - 1;
        if (rank > 0) wait_turn(cnt, rank, p.ctrl, p.spin_ticks, lane);
        const __amdgpu_buffer_rsrc_t racc =
            __builtin_amdgcn_make_buffer_rsrc(acc, 0, C::MQ * 4096, 0x00020000);
        // one 32-row block at a time keeps the live set small
#pragma unroll
        for (int m = 0; m < C::MQ; ++m) {
          const int am = (m * 4 * 64 + lane) * 16;  // byte offset in the slice
          if (rank > 0) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4 old = __builtin_amdgcn_raw_buffer_load_b128(racc, am + q4 * 1024, 0, kSC1);
#pragma unroll
              for (int e = 0; e < 4; ++e) dq[m][4 * q4 + e] = old[e] + dq[m][4 * q4 + e];
            }
          }
          if (!last) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4 x = {dq[m][4 * q4], dq[m][4 * q4 + 1], dq[m][4 * q4 + 2], dq[m][4 * q4 + 3]};
              __builtin_amdgcn_raw_buffer_store_b128(x, racc, am + q4 * 1024, 0, kSC1);
            }
          } else {
            // final value: dQ = scale * sum, bf16
            bf16* const gdq = (bf16*)p.dq;
            const int rs = p.Hq * D;
            const int base = (b * S + j * T) * rs + h * D + 32 * db + c;
            const int last_row = S - 1 - j * T;
            const bool full = (j + 1) * T <= S;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int ql = 32 * (qg * C::MQ + m) + 8 * (r >> 2) + 4 * hg + (r & 3);
              if (full || ql <= last_row) gdq[base + ql * rs] = (bf16)(dq[m][r] * p.scale);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // release: all of this wave's accumulator stores acknowledged first
        order_point();
        __builtin_amdgcn_s_waitcnt(0);
        order_point();
        if (lane == 0)
          __hip_atomic_store(cnt, rank + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
}

// ---------------------------------------------------------------------------
// Atomic reference only: dQ partial sums -> bf16 dq.  One thread per float of
// the accumulator, laid out as [tile][wave slice][row block m][r][lane].
template <int D, int T>
__global__ __launch_bounds__(256) void bwd_finalize(FinParams p) {
  constexpr int NW = T / 32, DB = D / 32, MQ = DB;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)p.B * p.Hq * p.N * NW * MQ * 16 * 64;
  if (idx >= total) return;
  const int lane = (int)(idx % 64);
  long long rest = idx / 64;
  const int r = (int)(rest % 16);
  rest /= 16;
  const int m = (int)(rest % MQ);
  rest /= MQ;
  const int w = (int)(rest % NW);
  rest /= NW;
  const int j = (int)(rest % p.N);
  const long long bh = rest / p.N;
  const int b = (int)(bh / p.Hq), h = (int)(bh % p.Hq);
  const int qg = w / DB, db = w % DB;
  const int ql = 32 * (qg * MQ + m) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
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
  const long long total = (long long)p.B * p.Hq * p.N * (T / 32) * (D / 32) * 16 * 64;
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
