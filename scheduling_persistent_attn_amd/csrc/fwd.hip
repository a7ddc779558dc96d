// Attention forward for gfx950: produces O (bf16) and the natural-log LSE
// (fp32) that the backward consumes.  Not part of the scheduled backward; one
// workgroup per (128-row query block, query head, batch), no cross-workgroup
// reduction, hence deterministic.
//
// Wave w owns query rows [32w, 32w+32) of the block.  Per 64-key block:
//   S^T  = K Q^T           A = K rows (LDS), B = Q fragments (registers)
//   online softmax over keys: each lane holds one query column of S^T, so the
//   row statistics are lane-local plus one exchange with lane ^ 32
//   O^T += V^T P^T         A = V^T (LDS, transposed), B = P^T (registers, the
//                          accumulator layout reused as the B operand)
// exp is computed as exp2 with the scale folded into log2(e).  Two workgroups
// per compute unit (the register budget is capped at two waves per SIMD), so
// one workgroup's loads overlap the other's products; with a causal mask the
// query blocks with the most key blocks are launched first.

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace dash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

__device__ __forceinline__ f32x16 mfma_f(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int CH>
__device__ __forceinline__ int rm_off_f(int row, int chunk) {
  constexpr int M = (CH < 16 ? CH : 16) - 1;
  return (row * CH + (chunk ^ (row & M))) * 8;
}
template <int C8>
__device__ __forceinline__ int tr_off_f(int d, int v) {
  const int sw = ((d & 15) ^ ((d >> 3) & 15)) & (C8 - 1);
  return (d * C8 + (v ^ sw)) * 4;
}

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd(FwdParams p) {
  constexpr int BQ = 128, BK = 64;
  constexpr int KBD = D / 16, DB = D / 32, CHD = D / 8, C8 = BK / 4;
  __shared__ __attribute__((aligned(16))) bf16 sK[BK * D];
  __shared__ __attribute__((aligned(16))) bf16 sVT[D * BK];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, c = lane & 31, hg = lane >> 5;
  // causal: the query blocks with the most key blocks first (the grid's
  // tail is then made of short blocks)
  const int qblk = CAUSAL ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int hk = h / p.G;
  const int S = p.S;
  const bf16* gq = (const bf16*)p.q;
  const bf16* gk = (const bf16*)p.k;
  const bf16* gv = (const bf16*)p.v;

  const int qrow = qblk * BQ + 32 * w + c;  // this lane's query row
  const bool q_ok = qrow < S;
  bf16x8 qB[KBD];
  {
    const int qr = q_ok ? qrow : S - 1;
    const bf16* src = gq + ((size_t)((size_t)b * S + qr) * p.Hq + h) * D + 8 * hg;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) qB[kb] = *reinterpret_cast<const bf16x8*>(src + 16 * kb);
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int md = 0; md < DB; ++md) oacc[md] = f32x16{};
  float m_run = -__builtin_inff();
  float l_part = 0.0f;

  const int kend = CAUSAL ? min(S, (qblk + 1) * BQ) : S;
  const int nblk = (kend + BK - 1) / BK;
  const int krs = p.Hkv * D;
  for (int kbk = 0; kbk < nblk; ++kbk) {
    __syncthreads();
    // K block row-major; V block transposed (4 keys x 8 features per unit)
    for (int un = tid; un < (BK / 4) * CHD; un += 256) {
      const int cu = un % CHD, rg = un / CHD;
      bf16x8 kr[4], vr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kbk * BK + 4 * rg + e;
        const int kc = key < S ? key : S - 1;
        const size_t off = ((size_t)((size_t)b * S + kc) * p.Hkv + hk) * D + 8 * cu;
        kr[e] = *reinterpret_cast<const bf16x8*>(gk + off);
        vr[e] = *reinterpret_cast<const bf16x8*>(gv + off);
        if (key >= S) {
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            kr[e][x] = (bf16)0.0f;
            vr[e][x] = (bf16)0.0f;
          }
        }
        *reinterpret_cast<bf16x8*>(sK + rm_off_f<CHD>(4 * rg + e, cu)) = kr[e];
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        bf16x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = vr[e][x];
        *reinterpret_cast<bf16x4*>(sVT + tr_off_f<C8>(8 * cu + x, rg)) = t;
      }
    }
    __syncthreads();

    f32x16 sacc[2];
#pragma unroll
    for (int mk = 0; mk < 2; ++mk) {
      sacc[mk] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + rm_off_f<CHD>(32 * mk + c, 2 * kb + hg));
        sacc[mk] = mfma_f(a, qB[kb], sacc[mk]);
      }
    }
    // scale, mask, block max
    float bmax = -__builtin_inff();
#pragma unroll
    for (int mk = 0; mk < 2; ++mk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbk * BK + 32 * mk + 8 * (r >> 2) + 4 * hg + (r & 3);
        float x = sacc[mk][r] * p.scale_log2e;
        if (key >= S || (CAUSAL && key > qrow)) x = -__builtin_inff();
        sacc[mk][r] = x;
        bmax = fmaxf(bmax, x);
      }
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float m_new = fmaxf(m_run, bmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int mk = 0; mk < 2; ++mk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(sacc[mk][r] - m_new);
        psum += pv;
        pb[mk][r >> 3][r & 7] = (bf16)pv;
      }
    }
    l_part = l_part * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int md = 0; md < DB; ++md) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[md][r] *= alpha;
    }
#pragma unroll
    for (int md = 0; md < DB; ++md) {
#pragma unroll
      for (int mk = 0; mk < 2; ++mk) {
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          const int k0 = 32 * mk + 16 * kq + 4 * hg;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(sVT + tr_off_f<C8>(32 * md + c, k0 >> 2));
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(sVT + tr_off_f<C8>(32 * md + c, (k0 >> 2) + 2));
          bf16x8 a;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            a[s] = lo[s];
            a[s + 4] = hi[s];
          }
          oacc[md] = mfma_f(a, pb[mk][kq], oacc[md]);
        }
      }
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
  const dim3 grid((p.S + 127) / 128, p.Hq, p.B);
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (D == 64) {
    if (causal) hipLaunchKernelGGL((attn_fwd<64, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd<64, false>), grid, dim3(256), 0, s, p);
  } else if (D == 128) {
    if (causal) hipLaunchKernelGGL((attn_fwd<128, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((attn_fwd<128, false>), grid, dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dash
