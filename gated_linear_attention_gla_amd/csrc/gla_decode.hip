// gla_decode.hip -- single-token recurrent decode step, streaming fp32 states.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "GLA mixer"
// (fixed dk x dv state per head, so inference costs O(1) per token) and
// section "Inference optimization on Trainium2" (the serving path reads and
// writes one fixed-size recurrent state per sequence for each new token).
//
// Per (n, h):  S <- lam S + k v^T  (in place),  o = S^T q  (updated state).
// The step is a pure HBM stream (each state is read once and written once),
// so there is no MFMA.  A workgroup owns every row of CB-th of the state's
// columns (CB = 1: the whole state); thread (cg, rp) owns the four columns
// 4 cg..4 cg+3 of that slice and the rows rp, rp + RP, ...  Each row segment
// is read with whole 16-byte vectors, and the readout's column sums stay in
// the workgroup: the RP row-phase partials are combined through LDS.
//
// Output epilogue (page section "GLA mixer": self-augmentation, Head RMSNorm,
// SiLU gate).  EPI = 1: a workgroup owns the whole state and normalises its
// row itself.  EPI = 2: each column slice writes o' = o + gate v (fp32) and
// the sum of squares of its columns to a workspace, and decode_norm_kernel
// then scales the rows (the normalisation needs all DV columns).
#include "gla_common.hpp"
#include "gla_internal.h"

namespace gla {

template <int DK, int DV, int RP, int EPI = 0, int CB = 1>
__global__ void __launch_bounds__((DV / 4 / CB) * RP) decode_kernel(DecodeArgs a) {
  constexpr int CGS = DV / 4;         // float4 column groups of a state row
  constexpr int CG = CGS / CB;        // ... of this workgroup's column slice
  static_assert(CGS % CB == 0, "column slices of whole float4 groups");
  static_assert(EPI != 1 || CB == 1, "the in-kernel epilogue normalises whole rows");
  static_assert(EPI != 2 || (CB > 1 && CB <= 4 && CG <= 16), "split epilogue: column slices of one wave's lanes");
  constexpr int NTHR = CG * RP;
  static_assert(NTHR >= DK, "one thread per q, k element");
  constexpr int RPT = (DK + RP - 1) / RP;  // rows per thread
  __shared__ float sq[DK];
  __shared__ float sk[DK];
  __shared__ float4 so[RP][CG];

  const int64_t nh = blockIdx.x / CB;
  const int64_t n = nh / a.H;
  const int64_t h = nh - n * a.H;
  const int tid = threadIdx.x;
  const int cs = (int)(blockIdx.x % CB) * CG;  // first column group of the slice
  const int cg = cs + tid % CG;
  const int rp = tid / CG;

  if (tid < DK) {
    const int64_t oq = n * a.sq_n + h * a.sq_h + tid;
    const int64_t ok = n * a.sk_n + h * a.sk_h + tid;
    if (a.in_f32) {
      sq[tid] = reinterpret_cast<const float*>(a.q)[oq];
      sk[tid] = reinterpret_cast<const float*>(a.k)[ok];
    } else {
      sq[tid] = bf16_to_f32(reinterpret_cast<const bf16_t*>(a.q)[oq]);
      sk[tid] = bf16_to_f32(reinterpret_cast<const bf16_t*>(a.k)[ok]);
    }
  }
  float4 vv;
  {
    const int64_t ov = n * a.sv_n + h * a.sv_h + 4 * cg;
    if (a.in_f32) {
      vv = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.v) + ov);
    } else {
      const bf16_t* p = reinterpret_cast<const bf16_t*>(a.v) + ov;
      vv = make_float4(bf16_to_f32(p[0]), bf16_to_f32(p[1]), bf16_to_f32(p[2]), bf16_to_f32(p[3]));
    }
  }
  const float lam = a.lam[h];
  f32x4* S = reinterpret_cast<f32x4*>(a.S + n * a.S_stride_n + h * (int64_t)DK * DV);

  // issue every state load of this thread before the first use
  f32x4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int d = rp + i * RP;
    if (d < DK) st[i] = __builtin_nontemporal_load(&S[d * CGS + cg]);
  }
  __syncthreads();  // sq, sk ready

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int d = rp + i * RP;
    if (d < DK) {
      const float kd = sk[d], qd = sq[d];
      f32x4 s = st[i];
      s[0] = fmaf(lam, s[0], kd * vv.x);
      s[1] = fmaf(lam, s[1], kd * vv.y);
      s[2] = fmaf(lam, s[2], kd * vv.z);
      s[3] = fmaf(lam, s[3], kd * vv.w);
      __builtin_nontemporal_store(s, &S[d * CGS + cg]);
      acc.x = fmaf(qd, s[0], acc.x);
      acc.y = fmaf(qd, s[1], acc.y);
      acc.z = fmaf(qd, s[2], acc.z);
      acc.w = fmaf(qd, s[3], acc.w);
    }
  }
  // epilogue gate sigmoid(q . (aug * k)), reduced by the first wave
  __shared__ float sgate;
  if constexpr (EPI != 0) {
    if (tid < 64) {
      float part = 0.0f;
      for (int d = tid; d < DK; d += 64) part = fmaf(sq[d] * a.aug[h * DK + d], sk[d], part);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
      if (tid == 0) sgate = 1.0f / (1.0f + expf(-part));
    }
  }
  so[rp][cg - cs] = acc;
  __syncthreads();
  static_assert(CG <= 64, "the first wave finishes the output");
  if (tid < 64) {
    const bool own = tid < CG;  // lanes that own a column group
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    if (own) {
      r = so[0][tid];
#pragma unroll
      for (int p = 1; p < RP; ++p) {
        const float4 u = so[p][tid];
        r.x += u.x; r.y += u.y; r.z += u.z; r.w += u.w;
      }
    }
    if constexpr (EPI == 2) {
      // o' = o + gate v for this slice's columns, to the workspace with the
      // slice's sum of squares (lanes without columns add zero)
      const float gt = sgate;
      if (own) {
        r.x = fmaf(gt, vv.x, r.x);
        r.y = fmaf(gt, vv.y, r.y);
        r.z = fmaf(gt, vv.z, r.z);
        r.w = fmaf(gt, vv.w, r.w);
        *reinterpret_cast<float4*>(a.ws + nh * (int64_t)DV + 4 * (cs + tid)) = r;
      }
      float ss = own ? r.x * r.x + r.y * r.y + r.z * r.z + r.w * r.w : 0.0f;
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
      if (tid == 0) a.ws[a.N * a.H * (int64_t)DV + nh * 4 + (int)(blockIdx.x % CB)] = ss;
      return;
    }
    if constexpr (EPI == 1) {
      // o' = o + gate v; Head RMSNorm over the DV columns held by this wave
      // (lanes without columns add zero); times gamma and SiLU(g)
      const float gt = sgate;
      if (own) {
        r.x = fmaf(gt, vv.x, r.x);
        r.y = fmaf(gt, vv.y, r.y);
        r.z = fmaf(gt, vv.z, r.z);
        r.w = fmaf(gt, vv.w, r.w);
      }
      float ss = r.x * r.x + r.y * r.y + r.z * r.z + r.w * r.w;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
      const float rstd = 1.0f / sqrtf(ss * (1.0f / DV) + a.eps);
      if (own) {
        const float4 gm = *reinterpret_cast<const float4*>(a.gamma + h * DV + 4 * tid);
        const int64_t og = n * a.sg_n + h * a.sg_h + 4 * tid;
        float4 gv;
        if (a.in_f32) {
          gv = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.gz) + og);
        } else {
          const bf16_t* p = reinterpret_cast<const bf16_t*>(a.gz) + og;
          gv = make_float4(bf16_to_f32(p[0]), bf16_to_f32(p[1]), bf16_to_f32(p[2]), bf16_to_f32(p[3]));
        }
        r.x = r.x * rstd * gm.x * (gv.x / (1.0f + expf(-gv.x)));
        r.y = r.y * rstd * gm.y * (gv.y / (1.0f + expf(-gv.y)));
        r.z = r.z * rstd * gm.z * (gv.z / (1.0f + expf(-gv.z)));
        r.w = r.w * rstd * gm.w * (gv.w / (1.0f + expf(-gv.w)));
      }
    }
    if (own) {
      const int64_t oo = n * a.so_n + h * a.so_h + 4 * (cs + tid);
      if (a.o_f32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + oo) = r;
      } else {
        bf16_t* p = reinterpret_cast<bf16_t*>(a.o) + oo;
        p[0] = f32_to_bf16(r.x);
        p[1] = f32_to_bf16(r.y);
        p[2] = f32_to_bf16(r.z);
        p[3] = f32_to_bf16(r.w);
      }
    }
  }
  (void)NTHR;
}

// Second kernel of the split epilogue (EPI = 2): y = o' rstd gamma_h SiLU(g)
// with rstd = 1 / sqrt(sum of the CB slices' squares / DV + eps); one thread
// per float4 column group of a state row, reading the workspace written by
// decode_kernel.
template <int DV, int CB>
__global__ void __launch_bounds__(256) decode_norm_kernel(DecodeArgs a) {
  constexpr int CGS = DV / 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nh = t / CGS;
  if (nh >= a.N * a.H) return;
  const int cg = (int)(t - nh * CGS);
  const int64_t n = nh / a.H;
  const int64_t h = nh - n * a.H;
  const float* ssq = a.ws + a.N * a.H * (int64_t)DV + nh * 4;
  float tot = 0.0f;
#pragma unroll
  for (int c = 0; c < CB; ++c) tot += ssq[c];
  const float rstd = 1.0f / sqrtf(tot * (1.0f / DV) + a.eps);
  float4 r = *reinterpret_cast<const float4*>(a.ws + nh * (int64_t)DV + 4 * cg);
  const float4 gm = *reinterpret_cast<const float4*>(a.gamma + h * DV + 4 * cg);
  const int64_t og = n * a.sg_n + h * a.sg_h + 4 * cg;
  float4 gv;
  if (a.in_f32) {
    gv = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.gz) + og);
  } else {
    const bf16_t* p = reinterpret_cast<const bf16_t*>(a.gz) + og;
    gv = make_float4(bf16_to_f32(p[0]), bf16_to_f32(p[1]), bf16_to_f32(p[2]), bf16_to_f32(p[3]));
  }
  r.x = r.x * rstd * gm.x * (gv.x / (1.0f + expf(-gv.x)));
  r.y = r.y * rstd * gm.y * (gv.y / (1.0f + expf(-gv.y)));
  r.z = r.z * rstd * gm.z * (gv.z / (1.0f + expf(-gv.z)));
  r.w = r.w * rstd * gm.w * (gv.w / (1.0f + expf(-gv.w)));
  const int64_t oo = n * a.so_n + h * a.so_h + 4 * cg;
  if (a.o_f32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + oo) = r;
  } else {
    bf16_t* p = reinterpret_cast<bf16_t*>(a.o) + oo;
    p[0] = f32_to_bf16(r.x);
    p[1] = f32_to_bf16(r.y);
    p[2] = f32_to_bf16(r.z);
    p[3] = f32_to_bf16(r.w);
  }
}

bool decode_supported(int dk, int dv) {
  return (dk == 96 && dv == 192) || (dk == 16 && dv == 32);
}

// Threads of one decode workgroup, and how many column slices (workgroups)
// serve each state.  The (96, 192) step streams three 64-column slices per
// state (16 column groups x 24 row phases, 4 rows per thread), which measured
// faster than a workgroup per state and than 12 or 48 row phases.  The fused
// step does the same when it has its workspace (the normalisation then runs
// as a second kernel); without one it normalises whole rows in one workgroup
// per state.  A launch covers at most 2^32 - 1 work-items: with 384 threads
// per slice, three slices fit up to 3,728,270 states (about 275 GB of fp32
// states); beyond that the step runs one 192-thread workgroup per state.
static int decode_threads(int dk, int dv, bool epi, int slices) {
  if (dk == 96 && dv == 192) return slices == 3 ? 16 * 24 : 48 * 4;
  (void)epi;
  return 8 * 8;
}

int decode_slices(int64_t states, int dk, int dv, bool epi, bool has_ws) {
  if (!decode_supported(dk, dv) || states < 1) return 0;
  if (dk == 96 && dv == 192 && (!epi || has_ws)) {
    const int64_t items = states * 3 * decode_threads(dk, dv, epi, 3);
    if (items <= (int64_t)0xFFFFFFFF) return 3;
  }
  return 1;
}

hipError_t launch_decode(int dk, int dv, const DecodeArgs& a, hipStream_t st) {
  const int64_t nblocks = a.N * a.H;
  if (nblocks <= 0) return hipSuccess;
  const bool epi = a.gz != nullptr;
  const int slices = decode_slices(nblocks, dk, dv, epi, a.ws != nullptr);
  if (slices == 0 || nblocks * slices * decode_threads(dk, dv, epi, slices) > (int64_t)0xFFFFFFFF)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(nblocks * slices)), block(decode_threads(dk, dv, epi, slices));
  if (dk == 96 && dv == 192) {
    if (epi && slices == 3) {
      hipLaunchKernelGGL((decode_kernel<96, 192, 24, 2, 3>), grid, block, 0, st, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t nthr = nblocks * (192 / 4);
      hipLaunchKernelGGL((decode_norm_kernel<192, 3>), dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st, a);
    } else if (epi) {
      hipLaunchKernelGGL((decode_kernel<96, 192, 4, 1>), grid, block, 0, st, a);
    } else if (slices == 3) {
      hipLaunchKernelGGL((decode_kernel<96, 192, 24, 0, 3>), grid, block, 0, st, a);
    } else {
      hipLaunchKernelGGL((decode_kernel<96, 192, 4>), grid, block, 0, st, a);
    }
  } else {
    if (epi) hipLaunchKernelGGL((decode_kernel<16, 32, 8, 1>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_kernel<16, 32, 8>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace gla
