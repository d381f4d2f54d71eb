/*
 * gla_epilogue_oracle.c -- fp64 CPU oracle of the mixer's output epilogue.
 *
 * TEST INFRASTRUCTURE ONLY (same rules as gla_oracle.c: loaded only by the
 * test suite, the package smoke check and the benchmark's CPU-baseline leg;
 * no code shared with the HIP library).
 *
 * Source: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
 * attention model on AWS Trainium2 with native PyTorch", section "GLA mixer",
 * the paragraphs after the readout: a self-augmentation step adds a gated
 * copy of the value to each head's output, the gate being the sigmoid of the
 * query-key dot product with a learned per-channel scale a ("aug_balance",
 * zero at initialisation, i.e. a half-strength skip of the value); the head
 * outputs then go through Head RMSNorm (one per decay tier), are
 * concatenated, gated by SiLU(g_t) and projected (the projection is not part
 * of this step).
 *
 * Readings (the equations were images): per token t and head h,
 *   o'  = o + sigmoid(sum_i q[i] a[h][i] k[i]) * v
 *   r   = o' / sqrt(mean_j o'[j]^2 + eps) * gamma[h]
 *   y   = r * SiLU(g),  SiLU(x) = x / (1 + exp(-x))
 * where gamma[h] is the RMSNorm weight of h's tier (the caller repeats a
 * tier's weight for each of its heads).  Layouts: q, k [B][H][T][dk];
 * v, o, g, y [B][H][T][dv]; a [H][dk]; gamma [H][dv].  Double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void gla_oracle_epilogue(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, const double* q,
                         const double* k, const double* v, const double* o, const double* a,
                         const double* gamma, double eps, const double* g, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const int64_t h = bh % H;
    double* op = (double*)malloc(sizeof(double) * (size_t)dv);
    for (int64_t t = 0; t < T; ++t) {
      const size_t rk = ((size_t)bh * T + t) * dk, rv = ((size_t)bh * T + t) * dv;
      /* self-augmentation gate */
      double s = 0.0;
      for (int64_t i = 0; i < dk; ++i) s += q[rk + i] * a[(size_t)h * dk + i] * k[rk + i];
      const double gate = 1.0 / (1.0 + exp(-s));
      double ms = 0.0;
      for (int64_t j = 0; j < dv; ++j) {
        op[j] = o[rv + j] + gate * v[rv + j];
        ms += op[j] * op[j];
      }
      /* Head RMSNorm over the head's dv channels */
      const double rstd = 1.0 / sqrt(ms / (double)dv + eps);
      for (int64_t j = 0; j < dv; ++j) {
        const double x = g[rv + j];
        y[rv + j] = op[j] * rstd * gamma[(size_t)h * dv + j] * (x / (1.0 + exp(-x)));
      }
    }
    free(op);
  }
}
