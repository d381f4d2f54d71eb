// gla_common.hpp -- CDNA4 (gfx950) building blocks shared by the Simple GLA
// kernels: bf16 vector types, the bf16 MFMA with multi-term operand splitting,
// LDS fragment loads (plain and transposing) and value conversions.
//
// Lane maps (measured on gfx950 and relied on throughout):
//   v_mfma_f32_16x16x32_bf16, lane l, g = l / 16:
//     A[m][k]:  m = l % 16, k = 8 g + e          (e = 0..7, one bf16x8)
//     B[k][n]:  n = l % 16, k = 8 g + e
//     D[m][n]:  n = l % 16, m = 4 g + r          (r = 0..3, one f32x4)
//   ds_read_b64_tr_b16 inside each 16-lane group: if lane s supplies the
//     address of four consecutive bf16 values src[s][0..3], lane i receives
//     { src[4e + i/4][i % 4] : e = 0..3 }.  With lane s pointing at
//     M[r0 + s/4][c0 + 4 (s % 4)] of a row-major tile, lane i receives
//     M[r0 + e][c0 + i], e = 0..3: a column read of a row-major tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) short lds_short;

typedef uint16_t bf16_t;  // raw storage type of bf16 in memory

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}
// Round-to-nearest-even float -> bf16 (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}
__device__ __forceinline__ float bf16v_to_f32(__bf16 b) {
  return bf16_to_f32(__builtin_bit_cast(bf16_t, b));
}

// Split x into NT bf16 terms with x ~= t0 + t1 + ... (each residual exact in fp32).
template <int NT>
__device__ __forceinline__ void split_terms(float x, __bf16 (&t)[NT]) {
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    t[i] = (__bf16)x;
    if (i + 1 < NT) x = x - bf16v_to_f32(t[i]);
  }
}

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Two-term split of a pair: hi = RNE(x), lo = RNE(x - hi), each pair packed
// with element 0 in the low half.  One packed conversion yields both hi
// values, and their fp32 values are the packed word shifted or masked, so a
// pair costs six VALU instructions (the same terms as split_terms<2>).
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){x0, x1}, bf16x2v));
  const float r0 = x0 - __uint_as_float(u << 16);
  const float r1 = x1 - __uint_as_float(u & 0xffff0000u);
  hi = u;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){r0, r1}, bf16x2v));
}

// x[0..N) -> NT bf16 term vectors t[p] (N = 4 or 8), pairwise for two terms.
template <int NT, int N, typename V>
__device__ __forceinline__ void split_vec(const float (&x)[N], V (&t)[NT]) {
  if constexpr (NT == 2) {
    uint32_t h[N / 2], l[N / 2];
#pragma unroll
    for (int p = 0; p < N / 2; ++p) split_pair(x[2 * p], x[2 * p + 1], h[p], l[p]);
    t[0] = __builtin_bit_cast(V, h);
    t[1] = __builtin_bit_cast(V, l);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      __bf16 s[NT];
      split_terms<NT>(x[e], s);
#pragma unroll
      for (int p = 0; p < NT; ++p) t[p][e] = s[p];
    }
  }
}

// c += A * B over all term pairs (ia, ib) with ia + ib < max(NA, NB): the
// products dropped are below the precision the longer operand carries.
template <int NA, int NB>
__device__ __forceinline__ void mma_split(f32x4& c, const bf16x8 (&a)[NA], const bf16x8 (&b)[NB]) {
  constexpr int N = NA > NB ? NA : NB;
#pragma unroll
  for (int ia = NA - 1; ia >= 0; --ia)
#pragma unroll
    for (int ib = NB - 1; ib >= 0; --ib)
      if (ia + ib < N) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ia], b[ib], c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x4 lds_read_b64(const bf16_t* p) {
  return *reinterpret_cast<const bf16x4*>(p);
}
// Transposing LDS read (see lane map above); p must be 8-byte aligned LDS.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16_t* p) {
  lds_i16x4* q = (lds_i16x4*)((lds_short*)(p));
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat4(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace gla
