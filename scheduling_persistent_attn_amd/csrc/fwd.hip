// Attention forward for gfx950: produces O (bf16) and the natural-log LSE
// (fp32) that the backward consumes.  Not part of the scheduled backward; one
// workgroup of 8 waves per (256-row query block, query head, batch), no
// cross-workgroup reduction, hence deterministic.
//
// Wave w owns query rows [32w, 32w+32) of the block.  Per 64-key block:
//   S^T  = K Q^T           A = K rows (LDS, 16-byte reads), B = Q fragments
//                          (registers, loaded once)
//   online softmax over keys: each lane holds one query column of S^T, so the
//   row statistics are lane-local plus one exchange with lane ^ 32
//   O^T += V^T P^T         A = V^T, read from row-major V in LDS by
//                          transposing reads (ds_read_b64_tr_b16); B = P^T
//                          (registers, the accumulator layout reused)
// K and V blocks are staged through registers: the next block's loads are in
// flight while the current block's products run.  exp is computed as exp2
// with the scale folded into one FMA; the mask is applied only on blocks that
// cross the diagonal or the end of the sequence; O is rescaled only when a
// row maximum outgrows the running reference point by more than 2^8.  One
// workgroup per compute unit (two waves per SIMD, the register budget capped
// to match), so each key/value block staged in LDS serves 256 query rows;
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd(FwdParams p) {
  constexpr int BQ = 256, NT = 512, BK = 64, RB = 2 * D;  // RB: bytes of one K or V row
  constexpr int KBD = D / 16, DB = D / 32, CHD = D / 8;
  constexpr int NLD = BK * CHD / NT;            // 16-byte chunks per thread per tile
  constexpr float kGrow = 8.0f;                 // log2 headroom before O is rescaled
  __shared__ __attribute__((aligned(16))) char sK[BK * RB];
  __shared__ __attribute__((aligned(16))) char sV[BK * RB];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63, c = lane & 31, hg = lane >> 5;
  const int g16 = lane >> 4, s16 = lane & 15;
  // Workgroups are dispatched in linear order.  Causal: grid (Hq, B, blocks),
  // the query blocks with the most key blocks first across all heads, so the
  // grid's tail is made of short blocks.  Full mask: grid (blocks, Hq, B), so
  // the workgroups in flight share the keys and values of a few heads.
  const int qblk = CAUSAL ? (int)gridDim.z - 1 - (int)blockIdx.z : (int)blockIdx.x;
  const int h = CAUSAL ? blockIdx.x : blockIdx.y, b = CAUSAL ? blockIdx.y : blockIdx.z;
  const int hk = h / p.G;
  const int S = p.S;
  const float c2 = p.scale_log2e;
  const bf16* gq = (const bf16*)p.q;
  const bf16* gk = (const bf16*)p.k;
  const bf16* gv = (const bf16*)p.v;

  const int qmin = qblk * BQ + 32 * w;  // first query row of this wave
  const int qrow = qmin + c;            // this lane's query row
  const bool q_ok = qrow < S;
  bf16x8 qB[KBD];
  {
    const int qr = q_ok ? qrow : S - 1;
    const bf16* src = gq + ((size_t)((size_t)b * S + qr) * p.Hq + h) * D + 8 * hg;
#pragma unroll
    for (int kb = 0; kb < KBD; ++kb) qB[kb] = *reinterpret_cast<const bf16x8*>(src + 16 * kb);
  }

  // per-lane LDS offsets: 16-byte reads of K row c, chunk 2kb + hg (A operand
  // of S^T); transposing reads of V rows 8h8 + 4hg + (s16 >> 2), features
  // 16(g16 & 1) + 4(s16 & 3) .. +3 (A operand of O^T, feature block md: XOR 64md)
  const int offA = lds_phys<RB>(c, hg);
  int offT[2];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8) {
    const int col = 16 * (g16 & 1) + 4 * (s16 & 3);
    offT[h8] = lds_phys<RB>(8 * h8 + 4 * hg + (s16 >> 2), col >> 3) + 2 * (col & 7);
  }
  // loader: chunk tid + NT e of a tile is row tid / CHD + e NT / CHD,
  // chunk tid % CHD.  Loads go through a buffer resource that ends at the
  // last key of the sequence, so rows past it read as zero.
  int ldo[NLD];
#pragma unroll
  for (int e = 0; e < NLD; ++e) ldo[e] = lds_phys<RB>((tid + NT * e) / CHD, tid % CHD);
  const int krs = p.Hkv * D;                                     // key stride (elements)
  const int voff = ((tid / CHD) * krs + 8 * (tid % CHD)) * 2;   // bytes
  const size_t head0 = ((size_t)b * S * p.Hkv + hk) * D;         // key 0 of this head
  auto load = [&](int k0, bf16x8* kr, bf16x8* vr) {
    const int nbytes = ((S - k0 - 1) * krs + D) * 2;  // through the last key's row
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(gk + head0 + (size_t)k0 * krs), 0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(gv + head0 + (size_t)k0 * krs), 0, nbytes, 0x00020000);
#pragma unroll
    for (int e = 0; e < NLD; ++e) {
      const int soff = e * (NT / CHD) * krs * 2;
      kr[e] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, voff, soff, 0));
      vr[e] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, soff, 0));
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int md = 0; md < DB; ++md) oacc[md] = f32x16{};
  float m_run = -__builtin_inff();  // running max, scaled (log2) units
  float l_part = 0.0f;

  const int kend = CAUSAL ? min(S, (qblk + 1) * BQ) : S;
  const int nblk = (kend + BK - 1) / BK;
  bf16x8 kr[NLD], vr[NLD];
  load(0, kr, vr);
  for (int kbk = 0; kbk < nblk; ++kbk) {
    const int k0 = kbk * BK;
#pragma unroll
    for (int e = 0; e < NLD; ++e) {
      *reinterpret_cast<bf16x8*>(sK + ldo[e]) = kr[e];
      *reinterpret_cast<bf16x8*>(sV + ldo[e]) = vr[e];
    }
    __syncthreads();  // block kbk is in LDS
    if (kbk + 1 < nblk) load(k0 + BK, kr, vr);  // in flight during the products

    {
      f32x16 sacc[2];
#pragma unroll
      for (int mk = 0; mk < 2; ++mk) {
        sacc[mk] = f32x16{};
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (offA ^ (32 * kb)) + 32 * mk * RB);
          sacc[mk] = mfma_f(a, qB[kb], sacc[mk]);
        }
      }
      // mask (only blocks that cross the diagonal or the end of the sequence)
      // and the block's row maximum, in raw units
      if ((CAUSAL && k0 + BK - 1 > qmin) || k0 + BK > S) {
        // element r of sacc[mk] is key k0 + 4hg + 32mk + 8(r >> 2) + (r & 3);
        // it is masked when that key is past the sequence or past the query
        const int lim = (CAUSAL ? min(qrow, S - 1) : S - 1) - k0 - 4 * hg;
#pragma unroll
        for (int mk = 0; mk < 2; ++mk) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * mk + 8 * (r >> 2) + (r & 3) > lim) sacc[mk][r] = -__builtin_inff();
        }
      }
      float smax = -__builtin_inff();
#pragma unroll
      for (int mk = 0; mk < 2; ++mk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) smax = fmaxf(smax, sacc[mk][r]);
      }
      smax = fmaxf(smax, __shfl_xor(smax, 32));
      // scaling by c2 > 0 is monotonic, so this is the maximum of the scaled
      // scores.  The reference point m_run moves only when some row of the
      // wave would exceed it by more than 2^kGrow; otherwise P may reach
      // 2^kGrow, which fp32 and bf16 carry without loss.  O and l use the same
      // reference point throughout, so the result is exact either way.
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
      bf16x8 pb[2][2];
#pragma unroll
      for (int mk = 0; mk < 2; ++mk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[mk][r], c2, -m_run));
          psum += pv;
          pb[mk][r >> 3][r & 7] = (bf16)pv;
        }
      }
      l_part += psum;
      // O^T += V^T P^T; the P^T accumulator layout holds keys 4hg + (0..3) and
      // 8 + 4hg + (0..3) of each 16-key step, which the transposing reads of
      // V rows deliver in the same order
#pragma unroll
      for (int md = 0; md < DB; ++md) {
#pragma unroll
        for (int mk = 0; mk < 2; ++mk) {
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
    }
    __syncthreads();  // every wave is done with block kbk
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
