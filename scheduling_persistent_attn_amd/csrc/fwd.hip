// Attention forward for gfx950: produces O (bf16) and the natural-log LSE
// (fp32) that the backward consumes.  Not part of the scheduled backward; one
// workgroup of 8 waves per (256-row query block, query head, batch), no
// cross-workgroup reduction, hence deterministic.
//
// Wave w owns query rows [32w, 32w+32) of the block.  Per 128-key block:
//   S^T  = K Q^T           A = K rows (LDS, 16-byte reads), B = Q fragments
//                          (registers, loaded once)
//   online softmax over keys: each lane holds one query column of S^T, so the
//   row statistics are lane-local plus one exchange with lane ^ 32
//   O^T += V^T P^T         A = V^T, read from row-major V in LDS by
//                          transposing reads (ds_read_b64_tr_b16); B = P^T
//                          (registers, the accumulator layout reused)
// K and V blocks go through a two-stage LDS ring filled by direct-to-LDS
// buffer loads: the next block's copies are in flight while the current
// block's products run, with one barrier per block.  The ring is unrolled by
// two so that every LDS access names its stage's array, which lets the
// compiler see that reads of one stage need not wait for copies into the
// other.  exp is computed as exp2
// with the scale folded into one FMA; the mask is applied only on blocks that
// cross the diagonal or the end of the sequence; O is rescaled only when a
// row maximum outgrows the running reference point by more than 2^8.  One
// workgroup per compute unit (two waves per SIMD, the register budget capped
// to match; the ring takes 128 KiB of LDS at D = 128), so each key/value
// block staged in LDS serves 256 query rows;
// with a causal mask the query blocks with the most key blocks are launched
// first.

#include <hip/hip_runtime.h>

#include "kernels.h"
#include "lds_layout.h"

namespace dash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

namespace {

__device__ __forceinline__ f32x16 mfma_f(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

typedef __attribute__((address_space(3))) void lds_void;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd(FwdParams p) {
  constexpr int BQ = 256, NT = 512, BK = 128, RB = 2 * D;
  constexpr int KBD = D / 16, DB = D / 32, NKB = BK / 32;  // 32-key blocks per key block
  constexpr int RPS = RB == 256 ? 1 : 2;                     // rows per 256-byte super-row
  constexpr int BLK = BK * RB / 1024;                        // 1 KB copy blocks per tile
  constexpr int NW = NT / 64;
  constexpr float kGrow = 8.0f;
  __shared__ __attribute__((aligned(1024))) char sK0[BK * RB];
  __shared__ __attribute__((aligned(1024))) char sV0[BK * RB];
  __shared__ __attribute__((aligned(1024))) char sK1[BK * RB];
  __shared__ __attribute__((aligned(1024))) char sV1[BK * RB];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);
  const int lane = tid & 63, c = lane & 31, hg = lane >> 5;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int qblk = CAUSAL ? (int)gridDim.z - 1 - (int)blockIdx.z : (int)blockIdx.x;
  const int h = CAUSAL ? blockIdx.x : blockIdx.y, b = CAUSAL ? blockIdx.y : blockIdx.z;
  const int hk = h / p.G;
  const int S = p.S;
  const float c2 = p.scale_log2e;
  const bf16* gq = (const bf16*)p.q;
  const bf16* gk = (const bf16*)p.k;
  const bf16* gv = (const bf16*)p.v;

  const int qmin = qblk * BQ + 32 * w;
  const int qrow = qmin + c;
  const bool q_ok = qrow < S;
  bf16x8 qB[KBD];
  {
    const int qr = q_ok ? qrow : S - 1;
    const bf16* src = gq + ((size_t)((size_t)b * S + qr) * p.Hq + h) * D + 8 * hg;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) qB[kb] = *reinterpret_cast<const bf16x8*>(src + 16 * kb);
  }
  const int offA = lds_phys<RB>(c, hg);
  int offT[2];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8) {
    const int col = 16 * (g16 & 1) + 4 * (s16 & 3);
    offT[h8] = lds_phys<RB>(8 * h8 + 4 * hg + (s16 >> 2), col >> 3) + 2 * (col & 7);
  }
  // direct-to-LDS copy: wave w fills 1 KB blocks w, w + NW, ...; the lane's
  // slot in its first block holds source (row0, chunk0), and the slot pattern
  // repeats every 4 NW super-rows
  int row0, chunk0;
  lds_slot_source<RB>(4 * w + (lane >> 4), lane & 15, &row0, &chunk0);
  const int krs = p.Hkv * D;
  const int voff = (row0 * krs + chunk0 * 8) * 2;
  const size_t head0 = ((size_t)b * S * p.Hkv + hk) * D;
  auto issue = [&](int k0, char* dk, char* dv) {
    const int nbytes = ((S - k0 - 1) * krs + D) * 2;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(gk + head0 + (size_t)k0 * krs), 0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(gv + head0 + (size_t)k0 * krs), 0, nbytes, 0x00020000);
#pragma unroll
    for (int e = 0; e < BLK / NW; ++e) {
      const int blk = w + e * NW;
      const int soff = e * 4 * NW * RPS * krs * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dk + blk * 1024), 16, voff, soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dv + blk * 1024), 16, voff, soff, 0, 0);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int md = 0; md < DB; ++md) oacc[md] = f32x16{};
  float m_run = -__builtin_inff();
  float l_part = 0.0f;

  const int kend = CAUSAL ? min(S, (qblk + 1) * BQ) : S;
  const int nblk = (kend + BK - 1) / BK;

  auto compute = [&](int k0, const char* sK, const char* sV) {
    f32x16 sacc[NKB];
#pragma unroll
    for (int mk = 0; mk < NKB; ++mk) {
      sacc[mk] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (offA ^ (32 * kb)) + 32 * mk * RB);
        sacc[mk] = mfma_f(a, qB[kb], sacc[mk]);
      }
    }
    if ((CAUSAL && k0 + BK - 1 > qmin) || k0 + BK > S) {
      const int lim = (CAUSAL ? min(qrow, S - 1) : S - 1) - k0 - 4 * hg;
#pragma unroll
      for (int mk = 0; mk < NKB; ++mk) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * mk + 8 * (r >> 2) + (r & 3) > lim) sacc[mk][r] = -__builtin_inff();
      }
    }
    float smax = -__builtin_inff();
#pragma unroll
    for (int mk = 0; mk < NKB; ++mk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[mk][r]);
    }
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    const float bm = smax * c2;
    if (__builtin_amdgcn_ballot_w64(bm > m_run + kGrow) != 0) {
      const float m_new = fmaxf(m_run, bm);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int md = 0; md < DB; ++md) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
      }
      m_run = m_new;
    }
    float psum = 0.0f;
    bf16x8 pb[NKB][2];
#pragma unroll
    for (int mk = 0; mk < NKB; ++mk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[mk][r], c2, -m_run));
        psum += pv;
        pb[mk][r >> 3][r & 7] = (bf16)pv;
      }
    }
    l_part += psum;
#pragma unroll
    for (int md = 0; md < DB; ++md) {
#pragma unroll
      for (int mk = 0; mk < NKB; ++mk) {
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const int rows = (32 * mk + 16 * kq) * RB;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(sV + ((offT[0] ^ (64 * md)) + rows)));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(sV + ((offT[1] ^ (64 * md)) + rows)));
          bf16x8 a;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            a[x] = lo[x];
            a[x + 4] = hi[x];
          }
          oacc[md] = mfma_f(a, pb[mk][kq], oacc[md]);
        }
      }
    }
  };

  // two-stage ring, unrolled by two so that every LDS access names its array
  issue(0, sK0, sV0);
  for (int kbk = 0; kbk < nblk; kbk += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of block kbk landed
    __syncthreads();                // every wave's; stage 1 no longer read
    if (kbk + 1 < nblk) issue((kbk + 1) * BK, sK1, sV1);
    compute(kbk * BK, sK0, sV0);
    if (kbk + 1 < nblk) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kbk + 2 < nblk) issue((kbk + 2) * BK, sK0, sV0);
      compute((kbk + 1) * BK, sK1, sV1);
    }
  }

  const float l = l_part + __shfl_xor(l_part, 32);
  const float inv = 1.0f / l;
  if (q_ok) {
    bf16* dst = (bf16*)p.o + ((size_t)((size_t)b * S + qrow) * p.Hq + h) * D;
#pragma unroll
    for (int md = 0; md < DB; ++md) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (bf16)(oacc[md][4 * q4 + e] * inv);
        *reinterpret_cast<bf16x4*>(dst + 32 * md + 8 * q4 + 4 * hg) = x;
      }
    }
    if (hg == 0)
      p.lse[((size_t)b * p.Hq + h) * S + qrow] = (m_run + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
  }
}

hipError_t launch_fwd(int D, bool causal, const FwdParams& p, hipStream_t s) {
  const int nq = (p.S + 255) / 256;  // 256-row query blocks
  const dim3 grid = causal ? dim3(p.Hq, p.B, nq) : dim3(nq, p.Hq, p.B);
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (D == 64) {
    if (causal) hipLaunchKernelGGL((attn_fwd<64, true>), grid, dim3(512), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd<64, false>), grid, dim3(512), 0, s, p);
  } else if (D == 128) {
    if (causal) hipLaunchKernelGGL((attn_fwd<128, true>), grid, dim3(512), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd<128, false>), grid, dim3(512), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dash
