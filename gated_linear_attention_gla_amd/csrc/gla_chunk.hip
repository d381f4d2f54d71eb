// gla_chunk.hip -- chunked Simple GLA recurrence on CDNA4 bf16 MFMA.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "Challenge 1"
// (inside a chunk the output is decay-masked linear attention plus the
// running state's contribution; the state then advances by the decay
// compounded over the chunk, and only that advance is sequential) and section
// "GLA mixer" (S_t = lam S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, per head).
//
// For a chunk of L tokens with local index i, j in [0, L) and state S on
// entry, in forward time:
//   O[i]  = lam^{i+1} (S^T q_i) + sum_{j<=i} lam^{i-j} (q_i . k_j) v_j
//   S    <- lam^L S + sum_j lam^{L-1-j} k_j v_j^T
// In reverse time (used by the backward) the window is j >= i, the mask is
// lam^{j-i}, the state enters with lam^{L-1-i} and advances with lam^{j+1}.
// Only non-negative powers lam^n, n <= chunk, are ever formed (fp32 table).
//
// One workgroup owns one (b, h) and a BN-wide block of state/output columns
// and walks the chunks in order, keeping its DK x BN slice of the fp32 state
// in MFMA accumulators.  Each wave owns NS strips of 16 columns.  Per chunk:
//   stage 0  q, k, v tiles -> LDS (bf16 planes; fp32 inputs become 3 planes)
//   stage 1  P^T = K Q^T tiles (causal half only), masked in fp32 -> LDS
//   stage 2  O = diag(row factors) Q S   (state split hi+lo as bf16)
//   stage 3  O += P V, store O
//   stage 4  S = lam^L S + (col factors * K)^T V  (scaled K split hi+lo)
// The split-operand products keep the state path at fp32-level accuracy; the
// masked P tile is rounded once to bf16 (three terms for fp32 inputs).
#include "gla_common.hpp"
#include "gla_internal.h"

namespace gla {

// lam^n for n >= 0 in fp32, computed in double; 0^0 = 1.
__device__ __forceinline__ float lam_pow_f32(float lam, int n) {
  if (n == 0) return 1.0f;
  if (lam == 0.0f) return 0.0f;
  if (lam == 1.0f) return 1.0f;
  return (float)exp2((double)n * log2((double)lam));
}

template <int NT>
__device__ __forceinline__ void store_planes8(bf16_t* dst0, int plane_stride, const float (&x)[8]) {
  // x -> NT bf16 planes, 16 bytes per plane
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = x[e];
      __bf16 t[NT];
      split_terms<NT>(r, t);
      v[e] = t[p];
    }
    *reinterpret_cast<bf16x8*>(dst0 + (size_t)p * plane_stride) = v;
  }
}

// Copies rows [0, L) of a (rows x COLS) global tile into LDS (row pitch PITCH,
// NT planes of ROWS*PITCH elements); rows in [L, ROWS) are zero-filled, and so
// are columns [COLS, COLSP).
template <int NT, int ROWS, int COLS, int COLSP, int PITCH, int NTHR>
__device__ __forceinline__ void stage_tile(bf16_t* lds, const void* gsrc, int64_t row_stride, int L,
                                           int in_f32, int tid) {
  constexpr int VPR = COLSP / 8;  // 8-element vectors per row
  constexpr int NVEC = ROWS * VPR;
  constexpr int PLANE = ROWS * PITCH;
  for (int idx = tid; idx < NVEC; idx += NTHR) {
    const int r = idx / VPR;
    const int c = (idx - r * VPR) * 8;
    bf16_t* dst = lds + r * PITCH + c;
    if (r < L && c < COLS) {
      if constexpr (NT == 1) {
        // bf16 input: raw 16-byte copy
        const bf16_t* src = reinterpret_cast<const bf16_t*>(gsrc) + (int64_t)r * row_stride + c;
        *reinterpret_cast<bf16x8*>(dst) = *reinterpret_cast<const bf16x8*>(src);
      } else {
        float x[8];
        if (in_f32) {
          const float* src = reinterpret_cast<const float*>(gsrc) + (int64_t)r * row_stride + c;
          const float4 a = *reinterpret_cast<const float4*>(src);
          const float4 b = *reinterpret_cast<const float4*>(src + 4);
          x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
          x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        } else {
          const bf16_t* src = reinterpret_cast<const bf16_t*>(gsrc) + (int64_t)r * row_stride + c;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(src[e]);
        }
        store_planes8<NT>(dst, PLANE, x);
      }
    } else {
      bf16x8 z;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
#pragma unroll
      for (int p = 0; p < NT; ++p) *reinterpret_cast<bf16x8*>(dst + p * PLANE) = z;
    }
  }
}

template <int DK, int DV, int BN, int NW, int C, int NT>
__global__ void __launch_bounds__(NW * 64) chunk_kernel(ChunkArgs a) {
  constexpr int NTHR = NW * 64;
  constexpr int NS = BN / (16 * NW);  // 16-column strips per wave
  static_assert(NS >= 1 && NS * 16 * NW == BN, "BN must split into 16-wide strips per wave");
  static_assert(DV % BN == 0, "DV must be a multiple of BN");
  static_assert(DK % 16 == 0 && C % 16 == 0, "dims must be multiples of 16");
  constexpr int NBLK = DV / BN;
  constexpr int CP = (C + 31) / 32 * 32;    // chunk rows padded to the 32-deep k-step
  constexpr int DKP = (DK + 31) / 32 * 32;  // DK padded likewise
  constexpr int NTP = NT == 3 ? 3 : 1;      // terms of the masked P tile
  constexpr int NTS = NT == 3 ? 3 : 2;      // terms of state fragments
  constexpr int NTK = NT == 3 ? 3 : 2;      // terms of decay-scaled keys
  constexpr int PQ = DKP + 8;               // LDS row pitches (elements)
  constexpr int PVV = BN + 8;
  constexpr int PP = CP + 8;
  constexpr int DKT = DK / 16;  // 16-row tiles of the state
  constexpr int KSD = DKP / 32;  // 32-deep k-steps over DK
  constexpr int CT = CP / 16;    // 16-row tiles of a chunk
  constexpr int KSC = CP / 32;   // 32-deep k-steps over the chunk

  __shared__ __attribute__((aligned(16))) bf16_t sQ[NT * CP * PQ];
  __shared__ __attribute__((aligned(16))) bf16_t sK[NT * CP * PQ];
  __shared__ __attribute__((aligned(16))) bf16_t sV[NT * CP * PVV];
  __shared__ __attribute__((aligned(16))) bf16_t sP[NTP * CP * PP];
  __shared__ float sPow[CP + 2];

  // XCD-aware block decode: consecutive dispatch slots on one XCD (block ids
  // congruent mod 8) walk the column blocks of the same (b, h), so the q/k
  // tiles they share are served from that XCD's L2.
  const int64_t BH = a.B * a.H;
  const int xb = blockIdx.x;
  const int xcd = xb & 7;
  const int slot = xb >> 3;
  const int64_t bh = (int64_t)(slot / NBLK) * 8 + xcd;
  const int nblk = slot % NBLK;
  if (bh >= BH) return;
  const int64_t b = bh / a.H;
  const int64_t h = bh - b * a.H;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int g = l >> 4;
  const int li = l & 15;
  const int rev = a.reverse;

  const float lam = a.lam[h];
  for (int n = tid; n <= CP + 1; n += NTHR) sPow[n] = lam_pow_f32(lam, n);

  const char* qb = reinterpret_cast<const char*>(a.q);
  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  const int esz = a.in_f32 ? 4 : 2;
  const int64_t q_off = b * a.sq_b + h * a.sq_h;
  const int64_t k_off = b * a.sk_b + h * a.sk_h;
  const int64_t v_off = b * a.sv_b + h * a.sv_h + (int64_t)nblk * BN;

  // column of this lane inside strip s (global state/output column)
  auto colof = [&](int s) { return nblk * BN + (w * NS + s) * 16 + li; };

  // ---- state slice in accumulators: accS[D][s][r] = S[16 D + 4 g + r][colof(s)]
  f32x4 accS[DKT][NS];
  {
    const float* si = a.s_init ? a.s_init + bh * (int64_t)DK * DV : nullptr;
#pragma unroll
    for (int D = 0; D < DKT; ++D)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 16 * D + 4 * g + r;
          const int n = colof(s);
          float x = 0.0f;
          if (si) x = a.s_init_trans ? si[(int64_t)n * DK + d] : si[(int64_t)d * DV + n];
          accS[D][s][r] = x;
        }
  }

  const int64_t T = a.T;
  const int64_t nchunks = (T + C - 1) / C;
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int64_t c = rev ? (nchunks - 1 - ci) : ci;
    const int64_t t0 = c * C;
    const int L = (int)((T - t0) < C ? (T - t0) : C);

    // ---------------- stage 0: tiles -> LDS
    stage_tile<NT, CP, DK, DKP, PQ, NTHR>(sQ, qb + (q_off + t0 * a.sq_t) * esz, a.sq_t, L, a.in_f32, tid);
    stage_tile<NT, CP, DK, DKP, PQ, NTHR>(sK, kb + (k_off + t0 * a.sk_t) * esz, a.sk_t, L, a.in_f32, tid);
    stage_tile<NT, CP, BN, BN, PVV, NTHR>(sV, vb + (v_off + t0 * a.sv_t) * esz, a.sv_t, L, a.in_f32, tid);
    __syncthreads();

    // ---------------- stage 1: masked P tiles (P[i][j] stored row-major)
    {
      int idx = 0;
#pragma unroll
      for (int I = 0; I < CT; ++I) {
#pragma unroll
        for (int J = 0; J < CT; ++J) {
          const bool need = rev ? (J >= I) : (J <= I);
          const bool zero = rev ? (J == I - 1 && (I & 1)) : (J == I + 1 && !(I & 1));
          if (!need && !zero) continue;
          if ((idx++ % NW) != w) continue;
          const int i = 16 * I + li;
          if (need) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
              bf16x8 A[NT], Bq[NT];
#pragma unroll
              for (int p = 0; p < NT; ++p) {
                A[p] = lds_read_b128(&sK[p * CP * PQ + (16 * J + li) * PQ + 32 * ks + 8 * g]);
                Bq[p] = lds_read_b128(&sQ[p * CP * PQ + i * PQ + 32 * ks + 8 * g]);
              }
              mma_split<NT, NT>(acc, A, Bq);
            }
            // acc[r] = q'_i . k'_j with j = 16 J + 4 g + r
            float val[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * J + 4 * g + r;
              const int diff = rev ? (j - i) : (i - j);
              val[r] = diff >= 0 ? acc[r] * sPow[diff] : 0.0f;
            }
#pragma unroll
            for (int p = 0; p < NTP; ++p) {
              bf16x4 pk;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                __bf16 t[NTP];
                split_terms<NTP>(val[r], t);
                pk[r] = t[p];
              }
              *reinterpret_cast<bf16x4*>(&sP[p * CP * PP + i * PP + 16 * J + 4 * g]) = pk;
            }
          } else {
            bf16x4 z;
#pragma unroll
            for (int r = 0; r < 4; ++r) z[r] = (__bf16)0.0f;
#pragma unroll
            for (int p = 0; p < NTP; ++p)
              *reinterpret_cast<bf16x4*>(&sP[p * CP * PP + i * PP + 16 * J + 4 * g]) = z;
          }
        }
      }
    }

    // ---------------- stage 2: O = diag(row factors) Q S
    f32x4 accO[CT][NS];
    {
      // State as the B operand of Q S: k-slot e of lane group g holds state
      // row 32 ks + 16 (e / 4) + 4 g + (e % 4), which is what the accumulator
      // layout already gives this lane; Q is read with the same permutation.
      bf16x8 Sf[KSD][NS][NTS];
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int D = 2 * ks + (e >> 2);
            const float x = (D < DKT) ? accS[D < DKT ? D : 0][s][e & 3] : 0.0f;
            __bf16 t[NTS];
            split_terms<NTS>(x, t);
#pragma unroll
            for (int p = 0; p < NTS; ++p) Sf[ks][s][p][e] = t[p];
          }
      const float cfac = sPow[L];
#pragma unroll
      for (int D = 0; D < DKT; ++D)
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int r = 0; r < 4; ++r) accS[D][s][r] *= cfac;

#pragma unroll
      for (int I = 0; I < CT; ++I) {
#pragma unroll
        for (int s = 0; s < NS; ++s) accO[I][s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          bf16x8 Aq[NT];
#pragma unroll
          for (int p = 0; p < NT; ++p) {
            const bf16_t* row = &sQ[p * CP * PQ + (16 * I + li) * PQ + 32 * ks];
            Aq[p] = cat4(lds_read_b64(row + 4 * g), lds_read_b64(row + 16 + 4 * g));
          }
#pragma unroll
          for (int s = 0; s < NS; ++s) mma_split<NT, NTS>(accO[I][s], Aq, Sf[ks][s]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * I + 4 * g + r;
          const float f = rev ? (i < L ? sPow[L - 1 - i] : 0.0f) : sPow[i + 1];
#pragma unroll
          for (int s = 0; s < NS; ++s) accO[I][s][r] *= f;
        }
      }
    }
    __syncthreads();  // P complete

    // ---------------- stage 3: O += P V ; stage 4: S += (colfac K)^T V
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      // V fragments: B[k = 32 ks + 8 g + e][n = strip col + li] via column reads
      bf16x8 Bv[NS][NT];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c0 = (w * NS + s) * 16 + 4 * (li & 3);
#pragma unroll
        for (int p = 0; p < NT; ++p) {
          const bf16_t* base = &sV[p * CP * PVV + (32 * ks + 8 * g + (li >> 2)) * PVV + c0];
          Bv[s][p] = cat4(lds_read_tr(base), lds_read_tr(base + 4 * PVV));
        }
      }
      // stage 3 for the row tiles whose causal window touches this k-step
#pragma unroll
      for (int I = 0; I < CT; ++I) {
        const bool use = rev ? (ks >= (I >> 1)) : (ks <= (I >> 1));
        if (!use) continue;
        bf16x8 Ap[NTP];
#pragma unroll
        for (int p = 0; p < NTP; ++p)
          Ap[p] = lds_read_b128(&sP[p * CP * PP + (16 * I + li) * PP + 32 * ks + 8 * g]);
#pragma unroll
        for (int s = 0; s < NS; ++s) mma_split<NTP, NT>(accO[I][s], Ap, Bv[s]);
      }
      // stage 4: decay-scaled keys as the A operand, A[m = d][k = j]
      float cf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * ks + 8 * g + e;
        cf[e] = (j < L) ? (rev ? sPow[j + 1] : sPow[L - 1 - j]) : 0.0f;
      }
#pragma unroll
      for (int D = 0; D < DKT; ++D) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
#pragma unroll
        for (int p = 0; p < NT; ++p) {
          const bf16_t* base = &sK[p * CP * PQ + (32 * ks + 8 * g + (li >> 2)) * PQ + 16 * D + 4 * (li & 3)];
          const bf16x8 raw = cat4(lds_read_tr(base), lds_read_tr(base + 4 * PQ));
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] += bf16v_to_f32(raw[e]);
        }
        bf16x8 Ak[NTK];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 t[NTK];
          split_terms<NTK>(x[e] * cf[e], t);
#pragma unroll
          for (int p = 0; p < NTK; ++p) Ak[p][e] = t[p];
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) mma_split<NTK, NT>(accS[D][s], Ak, Bv[s]);
      }
    }

    // store O rows < L
    {
      char* ob = reinterpret_cast<char*>(a.o);
#pragma unroll
      for (int I = 0; I < CT; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * I + 4 * g + r;
          if (i < L) {
            const int64_t rowoff = b * a.so_b + h * a.so_h + (t0 + i) * a.so_t;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              const int64_t off = rowoff + colof(s);
              if (a.o_f32) reinterpret_cast<float*>(ob)[off] = accO[I][s][r];
              else reinterpret_cast<bf16_t*>(ob)[off] = f32_to_bf16(accO[I][s][r]);
            }
          }
        }
    }
    __syncthreads();  // LDS reuse by the next chunk
  }

  if (a.s_final) {
    float* sf = a.s_final + bh * (int64_t)DK * DV;
#pragma unroll
    for (int D = 0; D < DKT; ++D)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) sf[(int64_t)(16 * D + 4 * g + r) * DV + colof(s)] = accS[D][s][r];
  }
}

template <int DK, int DV, int BN, int NW, int C, int NT>
static hipError_t launch_one(const ChunkArgs& a, hipStream_t st) {
  constexpr int NBLK = DV / BN;
  const int64_t BH = a.B * a.H;
  const int64_t groups = (BH + 7) / 8;
  const int64_t nblocks = groups * 8 * NBLK;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_kernel<DK, DV, BN, NW, C, NT>), dim3((unsigned)nblocks), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

// Tile shapes per (DK, DV): BN columns per workgroup, NW waves.
template <int DK, int DV, int C, int NT>
static hipError_t launch_shape(const ChunkArgs& a, hipStream_t st) {
  if constexpr (DK == 96 && DV == 192) return launch_one<96, 192, 96, 6, C, NT>(a, st);
  else if constexpr (DK == 192 && DV == 96) return launch_one<192, 96, 48, 3, C, NT>(a, st);
  else if constexpr (DK == 16 && DV == 32) return launch_one<16, 32, 32, 2, C, NT>(a, st);
  else if constexpr (DK == 32 && DV == 16) return launch_one<32, 16, 16, 1, C, NT>(a, st);
  else return hipErrorInvalidValue;
}

template <int DK, int DV, int NT>
static hipError_t launch_chunks(int chunk, const ChunkArgs& a, hipStream_t st) {
  switch (chunk) {
    case 16: return launch_shape<DK, DV, 16, NT>(a, st);
    case 32: return launch_shape<DK, DV, 32, NT>(a, st);
    case 64: return launch_shape<DK, DV, 64, NT>(a, st);
    case 128: return launch_shape<DK, DV, 128, NT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

bool chunk_pass_supported(int dk, int dv, int chunk, int in_f32) {
  if (!(chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128)) return false;
  const bool small = (dk == 16 && dv == 32) || (dk == 32 && dv == 16);
  const bool big = (dk == 96 && dv == 192) || (dk == 192 && dv == 96);
  if (!small && !big) return false;
  if (!in_f32) return true;
  // fp32 inputs keep three bf16 planes per tile in LDS; larger tiles exceed it
  if (small || dk == 96) return chunk <= 64;
  return chunk <= 32;
}

hipError_t launch_chunk_pass(int dk, int dv, int chunk, const ChunkArgs& a, hipStream_t st) {
  if (!a.in_f32) {
    if (dk == 96 && dv == 192) return launch_chunks<96, 192, 1>(chunk, a, st);
    if (dk == 192 && dv == 96) return launch_chunks<192, 96, 1>(chunk, a, st);
    if (dk == 16 && dv == 32) return launch_chunks<16, 32, 1>(chunk, a, st);
    if (dk == 32 && dv == 16) return launch_chunks<32, 16, 1>(chunk, a, st);
  } else {
    if (dk == 16 && dv == 32) {
      switch (chunk) {
        case 16: return launch_shape<16, 32, 16, 3>(a, st);
        case 32: return launch_shape<16, 32, 32, 3>(a, st);
        case 64: return launch_shape<16, 32, 64, 3>(a, st);
        default: return hipErrorInvalidValue;
      }
    }
    if (dk == 32 && dv == 16) {
      switch (chunk) {
        case 16: return launch_shape<32, 16, 16, 3>(a, st);
        case 32: return launch_shape<32, 16, 32, 3>(a, st);
        case 64: return launch_shape<32, 16, 64, 3>(a, st);
        default: return hipErrorInvalidValue;
      }
    }
    if (dk == 96 && dv == 192) {
      switch (chunk) {
        case 16: return launch_shape<96, 192, 16, 3>(a, st);
        case 32: return launch_shape<96, 192, 32, 3>(a, st);
        case 64: return launch_shape<96, 192, 64, 3>(a, st);
        default: return hipErrorInvalidValue;
      }
    }
    if (dk == 192 && dv == 96) {
      switch (chunk) {
        case 16: return launch_shape<192, 96, 16, 3>(a, st);
        case 32: return launch_shape<192, 96, 32, 3>(a, st);
        default: return hipErrorInvalidValue;
      }
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace gla
