// gla_conv.hip -- depthwise causal Conv1d (width 4) + SiLU in front of the
// mixer, for prefill/training and for the one-token decode step.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "i14 and
// Laplace 3B architecture", paragraph "Normalization and convolution": each
// channel of the residual stream is convolved causally over its last 4 tokens
// and passed through SiLU before the QKVG projection; the convolution window
// is part of a sequence's recurrent state.
//
//   z[t][c] = bias[c] + sum_{j<4} w[c][j] x[t-3+j][c],   y = z * sigmoid(z)
//
// Both kernels are HBM streams with no reuse beyond the 3-token window: a
// thread owns 8 adjacent channels (one 16-byte bf16 vector) and walks a run of
// tokens, keeping the window in registers, so every input row is read once
// (plus 3 rows per run) with fully coalesced 16-byte accesses.
#include "gla_common.hpp"
#include "gla_internal.h"

namespace gla {

namespace {

constexpr int CW = 4;        // convolution width
constexpr int CT = 16;       // tokens per thread run
constexpr int CTHR = 64;     // threads per wave (512 channels)
constexpr int RW = 4;        // prefill: waves per workgroup, one run each
static_assert(8 % RW == 0, "the tap staging splits 8 vectors per lane over the waves");

// 8 stored input values held between the load and their use (raw, so a bf16
// row costs 4 registers while its load is in flight)
template <bool F32> struct Raw8c;
template <> struct Raw8c<false> { bf16x8 v; };
template <> struct Raw8c<true> { f32x4 a, b; };

template <bool F32>
__device__ __forceinline__ void load_raw(const void* base, int64_t off, Raw8c<F32>& r) {
  if constexpr (F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + off);
    r.a = p[0];
    r.b = p[1];
  } else {
    r.v = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16_t*>(base) + off);
  }
}

template <bool F32>
__device__ __forceinline__ float raw_at(const Raw8c<F32>& r, int e) {
  if constexpr (F32) return e < 4 ? r.a[e] : r.b[e - 4];
  else return bf16v_to_f32(r.v[e]);
}

template <bool F32>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&v)[8]) {
  if constexpr (F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + off);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16_t*>(base) + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf16v_to_f32(a[e]);
  }
}

// outputs are not read again by these kernels: non-temporal stores
template <bool F32>
__device__ __forceinline__ void store8(void* base, int64_t off, const float (&v)[8]) {
  if constexpr (F32) {
    f32x4* p = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + off);
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, p);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, p + 1);
  } else {
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (__bf16)v[e];
    __builtin_nontemporal_store(a, reinterpret_cast<bf16x8*>(reinterpret_cast<bf16_t*>(base) + off));
  }
}

// SiLU with the hardware exponential and reciprocal (about 2 ulp each); for
// z -> -inf the reciprocal of +inf is 0, so the result tends to -0.
__device__ __forceinline__ float silu(float z) { return z * __frcp_rn(1.0f + __expf(-z)); }

// taps of 8 channels: wt[j][e] = w[c0 + e][j] (one 16-byte vector per
// channel, from global memory or from a workgroup's LDS copy); the bias as two
// 16-byte vectors (a lane's 8 biases are contiguous)
__device__ __forceinline__ void load_taps(const f32x4* w4, const float* bias, int64_t c0, float (&wt)[CW][8],
                                          float (&bs)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const f32x4 t = w4[e];
#pragma unroll
    for (int j = 0; j < CW; ++j) wt[j][e] = t[j];
  }
  f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = {0.f, 0.f, 0.f, 0.f};
  if (bias) {
    b0 = *reinterpret_cast<const f32x4*>(bias + c0);
    b1 = *reinterpret_cast<const f32x4*>(bias + c0 + 4);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bs[e] = b0[e];
    bs[4 + e] = b1[e];
  }
}

}  // namespace

// one thread = 8 channels x one run of CT tokens of one sequence
template <bool IN_F32, bool OUT_F32>
__global__ void __launch_bounds__(CTHR * RW) conv_fwd_kernel(ConvArgs a) {
  // Work items (sequence, channel block, group of RW consecutive runs), run
  // groups fastest, are dealt to the 8 XCDs in contiguous ranges: block ids
  // congruent mod 8 share an XCD, so the 3 window rows a run reads before its
  // first token were just read by the neighbouring run (another wave of the
  // workgroup, or the previous workgroup on the XCD) and come from L2.
  const int64_t cblocks = (a.D / 8 + CTHR - 1) / CTHR;
  const int64_t runs = a.T > 0 ? (a.T + CT - 1) / CT : 1;
  const int64_t rgroups = (runs + RW - 1) / RW;
  const int64_t items = a.B * rgroups * cblocks;
  const int64_t per_xcd = (items + 7) / 8;
  const int64_t bid = blockIdx.x;
  const int64_t item = (bid & 7) * per_xcd + (bid >> 3);
  if (item >= items) return;  // the padding of the last XCD's range (whole workgroup)
  const int tx = (int)threadIdx.x % CTHR;
  const int wr = (int)threadIdx.x / CTHR;  // this wave's run in the group
  const int64_t run = (item % rgroups) * RW + wr;
  const int64_t cb = (item / rgroups) % cblocks;
  const int64_t b = item / (rgroups * cblocks);
  const int64_t c0 = (cb * CTHR + tx) * 8;
  // The block's taps are staged in LDS once for its RW runs, with coalesced
  // loads: read directly, each lane's 128 contiguous bytes make every load
  // instruction touch 64 cache lines.  Every thread takes part, also those
  // past the last channel or run.
  __shared__ f32x4 sw[CTHR * 8];
  {
    const int64_t cbase = cb * CTHR * 8;
    const f32x4* wsrc = reinterpret_cast<const f32x4*>(a.w) + cbase;
#pragma unroll
    for (int k = 0; k < 8 / RW; ++k) {
      const int i = k * CTHR * RW + (int)threadIdx.x;
      if (cbase + i < a.D) sw[i] = wsrc[i];
    }
  }
  __syncthreads();
  if (c0 >= a.D || run >= runs) return;
  const int64_t t0 = run * CT;
  const int64_t t1 = (a.T - t0) < CT ? a.T : t0 + CT;
  float wt[CW][8], bs[8];

  // window: the 3 inputs before t0 (from x, else from the carried window)
  float h[CW - 1][8];
#pragma unroll
  for (int j = 0; j < CW - 1; ++j) {
    const int64_t s = t0 - (CW - 1) + j;
    if (s >= 0) {
      load8<IN_F32>(a.x, b * a.sx_b + s * a.sx_t + c0, h[j]);
    } else if (a.state_in) {
      const f32x4* p = reinterpret_cast<const f32x4*>(a.state_in + (b * (CW - 1) + (CW - 1 + s)) * a.D + c0);
      const f32x4 u = p[0], v = p[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[j][e] = u[e];
        h[j][4 + e] = v[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) h[j][e] = 0.0f;
    }
  }

  // tokens in groups of U, software-pipelined: the loads of group g + 1 are
  // in flight while group g is computed and stored
  constexpr int U = 4;
  constexpr int G = CT / U;
  Raw8c<IN_F32> xr[2][U];
  auto load_group = [&](int gi, Raw8c<IN_F32>(&dst)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + gi * U + u;
      if (t < t1) load_raw<IN_F32>(a.x, b * a.sx_b + t * a.sx_t + c0, dst[u]);
    }
  };
  load_group(0, xr[0]);
  load_taps(sw + tx * 8, a.bias, c0, wt, bs);
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    if (gi + 1 < G) load_group(gi + 1, xr[(gi + 1) & 1]);
    const int64_t t = t0 + gi * U;
    const Raw8c<IN_F32>(&xg)[U] = xr[gi & 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u < t1) {
        float yv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xe = raw_at<IN_F32>(xg[u], e);
          float z = bs[e];
          z = fmaf(wt[0][e], h[0][e], z);
          z = fmaf(wt[1][e], h[1][e], z);
          z = fmaf(wt[2][e], h[2][e], z);
          z = fmaf(wt[3][e], xe, z);
          yv[e] = silu(z);
          h[0][e] = h[1][e];
          h[1][e] = h[2][e];
          h[2][e] = xe;
        }
        store8<OUT_F32>(a.y, b * a.sy_b + (t + u) * a.sy_t + c0, yv);
      }
    }
  }
  // the run holding the last token hands the window on (T = 0: the carried one)
  if (a.state_out && t1 == a.T && (t0 < a.T || a.T == 0)) {
#pragma unroll
    for (int j = 0; j < CW - 1; ++j) {
      f32x4* p = reinterpret_cast<f32x4*>(a.state_out + (b * (CW - 1) + j) * a.D + c0);
      p[0] = f32x4{h[j][0], h[j][1], h[j][2], h[j][3]};
      p[1] = f32x4{h[j][4], h[j][5], h[j][6], h[j][7]};
    }
  }
}

// block id = sequence group * channel blocks + channel block; one token per
// sequence, window updated in place.  A thread serves SQ sequences of its 8
// channels so that their taps are loaded once: the windows and inputs (from
// HBM) are issued first, the taps (from L2) after them.
constexpr int SQ = 4;

template <bool IN_F32, bool OUT_F32>
__global__ void __launch_bounds__(CTHR) conv_step_kernel(ConvStepArgs a) {
  const int64_t cblocks = (a.D / 8 + CTHR - 1) / CTHR;
  const int64_t n0 = (blockIdx.x / cblocks) * SQ;
  const int64_t c0 = ((blockIdx.x % cblocks) * CTHR + threadIdx.x) * 8;
  if (c0 >= a.D) return;
  float h[SQ][CW - 1][8], xv[SQ][8];
#pragma unroll
  for (int i = 0; i < SQ; ++i) {
    const int64_t n = n0 + i;
    if (n < a.N) {
      const float* win = a.state + n * a.state_stride_n;
#pragma unroll
      for (int j = 0; j < CW - 1; ++j) {
        const f32x4* p = reinterpret_cast<const f32x4*>(win + j * a.D + c0);
        const f32x4 u = p[0], v = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[i][j][e] = u[e];
          h[i][j][4 + e] = v[e];
        }
      }
      load8<IN_F32>(a.x, n * a.sx_n + c0, xv[i]);
    }
  }
  float wt[CW][8], bs[8];
  load_taps(reinterpret_cast<const f32x4*>(a.w) + c0, a.bias, c0, wt, bs);
#pragma unroll
  for (int i = 0; i < SQ; ++i) {
    const int64_t n = n0 + i;
    if (n < a.N) {
      float yv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float z = bs[e];
        z = fmaf(wt[0][e], h[i][0][e], z);
        z = fmaf(wt[1][e], h[i][1][e], z);
        z = fmaf(wt[2][e], h[i][2][e], z);
        z = fmaf(wt[3][e], xv[i][e], z);
        yv[e] = silu(z);
      }
      store8<OUT_F32>(a.y, n * a.sy_n + c0, yv);
      // drop the oldest input, append this token
      float* win = a.state + n * a.state_stride_n;
#pragma unroll
      for (int j = 0; j < CW - 1; ++j) {
        const float* src = j + 1 < CW - 1 ? h[i][j + 1] : xv[i];
        f32x4* p = reinterpret_cast<f32x4*>(win + j * a.D + c0);
        p[0] = f32x4{src[0], src[1], src[2], src[3]};
        p[1] = f32x4{src[4], src[5], src[6], src[7]};
      }
    }
  }
}

int64_t conv_fwd_blocks(int64_t B, int64_t T, int64_t D) {
  const int64_t runs = T > 0 ? (T + CT - 1) / CT : 1;
  return (B * ((runs + RW - 1) / RW) * ((D / 8 + CTHR - 1) / CTHR) + 7) / 8 * 8;
}
int conv_fwd_threads() { return CTHR * RW; }

int64_t conv_step_blocks(int64_t N, int64_t D) { return (N + SQ - 1) / SQ * ((D / 8 + CTHR - 1) / CTHR); }
int conv_block_threads() { return CTHR; }

hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)conv_fwd_blocks(a.B, a.T, a.D)), block(CTHR * RW);
  if (a.in_f32) {
    if (a.out_f32) hipLaunchKernelGGL((conv_fwd_kernel<true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((conv_fwd_kernel<true, false>), grid, block, 0, st, a);
  } else {
    if (a.out_f32) hipLaunchKernelGGL((conv_fwd_kernel<false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((conv_fwd_kernel<false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_conv_step(const ConvStepArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)conv_step_blocks(a.N, a.D)), block(CTHR);
  if (a.in_f32) {
    if (a.out_f32) hipLaunchKernelGGL((conv_step_kernel<true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((conv_step_kernel<true, false>), grid, block, 0, st, a);
  } else {
    if (a.out_f32) hipLaunchKernelGGL((conv_step_kernel<false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((conv_step_kernel<false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace gla
