/* gla_abi_demo.c -- a plain C consumer of libgla.so (test infrastructure).
 *
 * Uses only include/gla.h and the HIP runtime's C API: device buffers from
 * hipMalloc, plain pointers and strides, the default stream.  Runs a chunked
 * forward (fp32, B=1, H=2, T=100, dk=16, dv=32, chunk 32, with S0 and S_T),
 * then one decode step from S_T, and checks both against the fp64 oracle
 * (liboracle.so, linked for this test only) to 1e-5 relative.  Then runs the
 * allocation-free forward on the same inputs (its results must equal the
 * workspace forward's bit for bit), and a fused decode step (fp32, N=3, H=2,
 * dk=96, dv=192) with its workspace against the oracle's decode step followed
 * by its epilogue.  Also checks that an invalid call is rejected with
 * GLA_ERR_NULL.  Exit status 0 on success.  Inputs come from splitmix64, a
 * counter-based generator, and are handed to both sides. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>

#include "gla.h"

/* oracle entry points (oracle/gla_oracle.c) */
void gla_oracle_fwd(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, const double* q, const double* k,
                    const double* v, const double* lam, const double* S0, double* o, double* S_T);
void gla_oracle_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv, const double* q, const double* k,
                            const double* v, const double* lam, double* S, double* o);
void gla_oracle_epilogue(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, const double* q,
                         const double* k, const double* v, const double* o, const double* a,
                         const double* gamma, double eps, const double* g, double* y);

static uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

/* uniform in [-scale, scale), exactly representable in fp32 */
static void fill(float* x, size_t n, uint64_t stream, float scale) {
  for (size_t i = 0; i < n; ++i) {
    const uint64_t r = splitmix64((stream << 40) ^ i) >> 40; /* 24 bits */
    x[i] = scale * ((float)r / 8388608.0f - 1.0f);
  }
}

static double max_rel(const float* got, const double* ref, size_t n) {
  double e = 0.0, m = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double d = fabs((double)got[i] - ref[i]);
    if (d > e) e = d;
    if (fabs(ref[i]) > m) m = fabs(ref[i]);
  }
  return m > 0.0 ? e / m : e;
}

#define CHECK_HIP(x)                                                  \
  do {                                                                \
    hipError_t err_ = (x);                                            \
    if (err_ != hipSuccess) {                                         \
      fprintf(stderr, "HIP error %d at line %d\n", (int)err_, __LINE__); \
      return 2;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  enum { B = 1, H = 2, T = 100, DK = 16, DV = 32, CHUNK = 32 };
  const size_t nq = (size_t)B * H * T * DK, nv = (size_t)B * H * T * DV, ns = (size_t)B * H * DK * DV;
  float *hq = malloc(nq * 4), *hk = malloc(nq * 4), *hv = malloc(nv * 4), *hS0 = malloc(ns * 4);
  float *ho = malloc(nv * 4), *hST = malloc(ns * 4), hlam[H] = {0.9f, 0.99f};
  fill(hq, nq, 1, 1.0f);
  fill(hk, nq, 2, 0.25f);
  fill(hv, nv, 3, 1.0f);
  fill(hS0, ns, 4, 0.01f);

  float *q, *k, *v, *o, *lam, *S0, *S_T;
  CHECK_HIP(hipMalloc((void**)&q, nq * 4));
  CHECK_HIP(hipMalloc((void**)&k, nq * 4));
  CHECK_HIP(hipMalloc((void**)&v, nv * 4));
  CHECK_HIP(hipMalloc((void**)&o, nv * 4));
  CHECK_HIP(hipMalloc((void**)&lam, H * 4));
  CHECK_HIP(hipMalloc((void**)&S0, ns * 4));
  CHECK_HIP(hipMalloc((void**)&S_T, ns * 4));
  CHECK_HIP(hipMemcpy(q, hq, nq * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k, hk, nq * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, hv, nv * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(lam, hlam, H * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(S0, hS0, ns * 4, hipMemcpyHostToDevice));

  /* dense [B, H, T, d] views */
  gla_dims dims = {B, H, T, DK, DV, CHUNK};
  gla_tensor tq = {q, GLA_F32, (int64_t)H * T * DK, (int64_t)T * DK, DK};
  gla_tensor tk = {k, GLA_F32, (int64_t)H * T * DK, (int64_t)T * DK, DK};
  gla_tensor tv = {v, GLA_F32, (int64_t)H * T * DV, (int64_t)T * DV, DV};
  gla_tensor to = {o, GLA_F32, (int64_t)H * T * DV, (int64_t)T * DV, DV};

  if (gla_chunk_fwd(&dims, NULL, &tk, &tv, lam, S0, &to, S_T, NULL, 0, NULL) != GLA_ERR_NULL) {
    fprintf(stderr, "a NULL query was not rejected\n");
    return 1;
  }
  const size_t nws = gla_chunk_fwd_workspace(&dims);
  void* ws = NULL;
  if (nws) CHECK_HIP(hipMalloc(&ws, nws));
  gla_status st = gla_chunk_fwd(&dims, &tq, &tk, &tv, lam, S0, &to, S_T, ws, nws, NULL);
  if (st != GLA_OK) {
    fprintf(stderr, "gla_chunk_fwd: %s\n", gla_status_string(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(ho, o, nv * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hST, S_T, ns * 4, hipMemcpyDeviceToHost));

  /* oracle on the same values, widened to fp64 */
  double *dq = malloc(nq * 8), *dk = malloc(nq * 8), *dv = malloc(nv * 8), *dS0 = malloc(ns * 8);
  double *ro = malloc(nv * 8), *rS = malloc(ns * 8), dlam[H];
  for (size_t i = 0; i < nq; ++i) { dq[i] = hq[i]; dk[i] = hk[i]; }
  for (size_t i = 0; i < nv; ++i) dv[i] = hv[i];
  for (size_t i = 0; i < ns; ++i) dS0[i] = hS0[i];
  for (int h = 0; h < H; ++h) dlam[h] = hlam[h];
  gla_oracle_fwd(B, H, T, DK, DV, dq, dk, dv, dlam, dS0, ro, rS);
  const double eo = max_rel(ho, ro, nv), eS = max_rel(hST, rS, ns);

  /* one decode step from S_T: N = 1 sequence, q/k/v of a fresh token ([N, H, d]) */
  float hq1[H * DK], hk1[H * DK], hv1[H * DV], ho1[H * DV], hS1[H * DK * DV];
  fill(hq1, H * DK, 5, 1.0f);
  fill(hk1, H * DK, 6, 0.25f);
  fill(hv1, H * DV, 7, 1.0f);
  float *q1, *k1, *v1, *o1;
  CHECK_HIP(hipMalloc((void**)&q1, sizeof hq1));
  CHECK_HIP(hipMalloc((void**)&k1, sizeof hk1));
  CHECK_HIP(hipMalloc((void**)&v1, sizeof hv1));
  CHECK_HIP(hipMalloc((void**)&o1, sizeof ho1));
  CHECK_HIP(hipMemcpy(q1, hq1, sizeof hq1, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k1, hk1, sizeof hk1, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v1, hv1, sizeof hv1, hipMemcpyHostToDevice));
  gla_tensor dq1 = {q1, GLA_F32, H * DK, DK, 0}, dk1 = {k1, GLA_F32, H * DK, DK, 0};
  gla_tensor dv1 = {v1, GLA_F32, H * DV, DV, 0}, do1 = {o1, GLA_F32, H * DV, DV, 0};
  st = gla_decode_step(1, H, DK, DV, &dq1, &dk1, &dv1, lam, S_T, (int64_t)H * DK * DV, &do1, NULL);
  if (st != GLA_OK) {
    fprintf(stderr, "gla_decode_step: %s\n", gla_status_string(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(ho1, o1, sizeof ho1, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hS1, S_T, sizeof hS1, hipMemcpyDeviceToHost));
  double dq1d[H * DK], dk1d[H * DK], dv1d[H * DV], ro1[H * DV];
  for (int i = 0; i < H * DK; ++i) { dq1d[i] = hq1[i]; dk1d[i] = hk1[i]; }
  for (int i = 0; i < H * DV; ++i) dv1d[i] = hv1[i];
  gla_oracle_decode_step(1, H, DK, DV, dq1d, dk1d, dv1d, dlam, rS, ro1); /* rS advances in place */
  const double eo1 = max_rel(ho1, ro1, H * DV), eS1 = max_rel(hS1, rS, ns);

  /* the allocation-free forward on the same inputs: equal to the workspace one */
  float *o2, *S_T2, *ho2 = malloc(nv * 4), *hST2 = malloc(ns * 4);
  CHECK_HIP(hipMalloc((void**)&o2, nv * 4));
  CHECK_HIP(hipMalloc((void**)&S_T2, ns * 4));
  gla_tensor to2 = {o2, GLA_F32, (int64_t)H * T * DV, (int64_t)T * DV, DV};
  st = gla_chunk_fwd_noalloc(&dims, &tq, &tk, &tv, lam, S0, &to2, S_T2, NULL);
  if (st != GLA_OK) {
    fprintf(stderr, "gla_chunk_fwd_noalloc: %s\n", gla_status_string(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(ho2, o2, nv * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hST2, S_T2, ns * 4, hipMemcpyDeviceToHost));
  int same = 1;
  for (size_t i = 0; i < nv; ++i) same &= ho2[i] == ho[i];
  for (size_t i = 0; i < ns; ++i) same &= hST2[i] == hST[i];

  /* a fused decode step at (96, 192) with its workspace */
  enum { N3 = 3, DK3 = 96, DV3 = 192 };
  const size_t n3q = (size_t)N3 * H * DK3, n3v = (size_t)N3 * H * DV3, n3s = (size_t)N3 * H * DK3 * DV3;
  float *h3q = malloc(n3q * 4), *h3k = malloc(n3q * 4), *h3v = malloc(n3v * 4), *h3g = malloc(n3v * 4);
  float *h3S = malloc(n3s * 4), *h3y = malloc(n3v * 4), *h3a = malloc(H * DK3 * 4), *h3gm = malloc(H * DV3 * 4);
  fill(h3q, n3q, 8, 1.0f);
  fill(h3k, n3q, 9, 0.1f);
  fill(h3v, n3v, 10, 1.0f);
  fill(h3g, n3v, 11, 2.0f);
  fill(h3S, n3s, 12, 0.01f);
  fill(h3a, H * DK3, 13, 0.2f);
  fill(h3gm, H * DV3, 14, 0.1f);
  for (int i = 0; i < H * DV3; ++i) h3gm[i] += 1.0f;
  float *q3, *k3, *v3, *g3, *S3, *y3, *a3, *gm3;
  CHECK_HIP(hipMalloc((void**)&q3, n3q * 4));
  CHECK_HIP(hipMalloc((void**)&k3, n3q * 4));
  CHECK_HIP(hipMalloc((void**)&v3, n3v * 4));
  CHECK_HIP(hipMalloc((void**)&g3, n3v * 4));
  CHECK_HIP(hipMalloc((void**)&S3, n3s * 4));
  CHECK_HIP(hipMalloc((void**)&y3, n3v * 4));
  CHECK_HIP(hipMalloc((void**)&a3, H * DK3 * 4));
  CHECK_HIP(hipMalloc((void**)&gm3, H * DV3 * 4));
  CHECK_HIP(hipMemcpy(q3, h3q, n3q * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k3, h3k, n3q * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v3, h3v, n3v * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(g3, h3g, n3v * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(S3, h3S, n3s * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(a3, h3a, H * DK3 * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(gm3, h3gm, H * DV3 * 4, hipMemcpyHostToDevice));
  const size_t nws3 = gla_decode_step_fused_workspace(N3, H, DK3, DV3);
  if (nws3 == 0) {
    fprintf(stderr, "the fused decode step reports no workspace at (96, 192)\n");
    return 1;
  }
  void* ws3;
  CHECK_HIP(hipMalloc(&ws3, nws3));
  gla_tensor t3q = {q3, GLA_F32, H * DK3, DK3, 0}, t3k = {k3, GLA_F32, H * DK3, DK3, 0};
  gla_tensor t3v = {v3, GLA_F32, H * DV3, DV3, 0}, t3g = {g3, GLA_F32, H * DV3, DV3, 0};
  gla_tensor t3y = {y3, GLA_F32, H * DV3, DV3, 0};
  const float eps = 1e-6f;
  st = gla_decode_step_fused(N3, H, DK3, DV3, &t3q, &t3k, &t3v, lam, S3, (int64_t)H * DK3 * DV3, &t3g, a3, gm3, eps,
                             &t3y, ws3, nws3, NULL);
  if (st != GLA_OK) {
    fprintf(stderr, "gla_decode_step_fused: %s\n", gla_status_string(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(h3y, y3, n3v * 4, hipMemcpyDeviceToHost));
  double *d3q = malloc(n3q * 8), *d3k = malloc(n3q * 8), *d3v = malloc(n3v * 8), *d3g = malloc(n3v * 8);
  double *d3S = malloc(n3s * 8), *d3o = malloc(n3v * 8), *d3y = malloc(n3v * 8);
  double *d3a = malloc(H * DK3 * 8), *d3gm = malloc(H * DV3 * 8);
  for (size_t i = 0; i < n3q; ++i) { d3q[i] = h3q[i]; d3k[i] = h3k[i]; }
  for (size_t i = 0; i < n3v; ++i) { d3v[i] = h3v[i]; d3g[i] = h3g[i]; }
  for (size_t i = 0; i < n3s; ++i) d3S[i] = h3S[i];
  for (int i = 0; i < H * DK3; ++i) d3a[i] = h3a[i];
  for (int i = 0; i < H * DV3; ++i) d3gm[i] = h3gm[i];
  gla_oracle_decode_step(N3, H, DK3, DV3, d3q, d3k, d3v, dlam, d3S, d3o);
  /* one token per sequence: [N, H, 1, d] is the [B, H, T, d] layout with T = 1 */
  gla_oracle_epilogue(N3, H, 1, DK3, DV3, d3q, d3k, d3v, d3o, d3a, d3gm, (double)eps, d3g, d3y);
  const double ey3 = max_rel(h3y, d3y, n3v);

  printf("abi %d  fwd: o %.3e  S_T %.3e   decode: o %.3e  S %.3e   noalloc equal: %d   fused decode: y %.3e\n",
         gla_abi_version(), eo, eS, eo1, eS1, same, ey3);
  const int ok = eo <= 1e-5 && eS <= 1e-5 && eo1 <= 1e-5 && eS1 <= 1e-5 && same && ey3 <= 1e-5;
  hipFree(o2); hipFree(S_T2); hipFree(q3); hipFree(k3); hipFree(v3); hipFree(g3); hipFree(S3); hipFree(y3);
  hipFree(a3); hipFree(gm3); hipFree(ws3);
  free(ho2); free(hST2); free(h3q); free(h3k); free(h3v); free(h3g); free(h3S); free(h3y); free(h3a); free(h3gm);
  free(d3q); free(d3k); free(d3v); free(d3g); free(d3S); free(d3o); free(d3y); free(d3a); free(d3gm);
  hipFree(q); hipFree(k); hipFree(v); hipFree(o); hipFree(lam); hipFree(S0); hipFree(S_T);
  hipFree(q1); hipFree(k1); hipFree(v1); hipFree(o1);
  if (ws) hipFree(ws);
  free(hq); free(hk); free(hv); free(hS0); free(ho); free(hST);
  free(dq); free(dk); free(dv); free(dS0); free(ro); free(rS);
  return ok ? 0 : 1;
}
