/*
 * gla_oracle.c -- fp64 CPU oracle for the Simple GLA mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg load this library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * Source: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
 * attention model on AWS Trainium2 with native PyTorch", section "GLA mixer"
 * (per-head matrix state of size dk x dv, fixed per-head decay lambda_h,
 * rank-1 write of the current key/value pair, readout of the state by the
 * query), section "Challenge 1" (chunked form: masked linear attention inside
 * a chunk plus the running state; the state advances by the decay compounded
 * over the chunk) and section "Challenge 3" (the backward pass differentiates
 * through the sequential state updates).
 *
 * The equations on that page were images that did not survive; the readings
 * used here (each documented in the design notes) are:
 *   S_t = lam * S_{t-1} + k_t v_t^T            (t = 1..T, S_0 given or zero)
 *   o_t = S_t^T q_t                            (readout of the updated state)
 * Everything is computed in double precision from inputs widened exactly.
 * Arrays are dense row-major: q,k [B][H][T][dk], v,o,dO [B][H][T][dv],
 * states [B][H][dk][dv], lam [H].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX3(t, d, D) ((size_t)(t) * (size_t)(D) + (size_t)(d))

/* pow with the convention 0^0 = 1 (C's pow already returns 1 for y == 0). */
static double lam_pow(double lam, int64_t n) { return pow(lam, (double)n); }

/* Token-by-token recurrence (the primary forward definition).
 * o: [B][H][T][dv]; S_T may be NULL; S0 may be NULL (zero state). */
void gla_oracle_fwd(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                    const double* q, const double* k, const double* v,
                    const double* lam, const double* S0, double* o, double* S_T) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const int64_t h = bh % H;
    const double l = lam[h];
    const double* qb = q + (size_t)bh * T * dk;
    const double* kb = k + (size_t)bh * T * dk;
    const double* vb = v + (size_t)bh * T * dv;
    double* ob = o + (size_t)bh * T * dv;
    double* S = (double*)malloc(sizeof(double) * dk * dv);
    if (S0) memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
    else memset(S, 0, sizeof(double) * dk * dv);
    for (int64_t t = 0; t < T; ++t) {
      /* state update: decay the old state, add the rank-1 write */
      for (int64_t i = 0; i < dk; ++i) {
        const double ki = kb[IDX3(t, i, dk)];
        for (int64_t j = 0; j < dv; ++j)
          S[IDX3(i, j, dv)] = l * S[IDX3(i, j, dv)] + ki * vb[IDX3(t, j, dv)];
      }
      /* readout of the updated state by the query */
      for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < dk; ++i) acc += qb[IDX3(t, i, dk)] * S[IDX3(i, j, dv)];
        ob[IDX3(t, j, dv)] = acc;
      }
    }
    if (S_T) memcpy(S_T + (size_t)bh * dk * dv, S, sizeof(double) * dk * dv);
    free(S);
  }
}

/* Brute-force quadratic form (self-check of the recurrence):
 *   o_t = lam^t S0^T q_t + sum_{s<=t} lam^{t-s} (q_t . k_s) v_s   (1-indexed t). */
void gla_oracle_fwd_bruteforce(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                               const double* q, const double* k, const double* v,
                               const double* lam, const double* S0, double* o) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const int64_t h = bh % H;
    const double l = lam[h];
    const double* qb = q + (size_t)bh * T * dk;
    const double* kb = k + (size_t)bh * T * dk;
    const double* vb = v + (size_t)bh * T * dv;
    const double* Sb = S0 ? S0 + (size_t)bh * dk * dv : NULL;
    double* ob = o + (size_t)bh * T * dv;
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t j = 0; j < dv; ++j) ob[IDX3(t, j, dv)] = 0.0;
      if (Sb) {
        const double w = lam_pow(l, t + 1);
        for (int64_t j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int64_t i = 0; i < dk; ++i) acc += qb[IDX3(t, i, dk)] * Sb[IDX3(i, j, dv)];
          ob[IDX3(t, j, dv)] += w * acc;
        }
      }
      for (int64_t s = 0; s <= t; ++s) {
        double qk = 0.0;
        for (int64_t i = 0; i < dk; ++i) qk += qb[IDX3(t, i, dk)] * kb[IDX3(s, i, dk)];
        const double w = lam_pow(l, t - s) * qk;
        for (int64_t j = 0; j < dv; ++j) ob[IDX3(t, j, dv)] += w * vb[IDX3(s, j, dv)];
      }
    }
  }
}

/* Closed form of the final state: S_T = lam^T S0 + sum_s lam^{T-s} k_s v_s^T. */
void gla_oracle_state_closed_form(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                  const double* k, const double* v, const double* lam,
                                  const double* S0, double* S_T) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const int64_t h = bh % H;
    const double l = lam[h];
    const double* kb = k + (size_t)bh * T * dk;
    const double* vb = v + (size_t)bh * T * dv;
    double* Sb = S_T + (size_t)bh * dk * dv;
    const double w0 = lam_pow(l, T);
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j)
        Sb[IDX3(i, j, dv)] = S0 ? w0 * S0[(size_t)bh * dk * dv + IDX3(i, j, dv)] : 0.0;
    for (int64_t s = 0; s < T; ++s) {
      const double w = lam_pow(l, T - 1 - s); /* 0-indexed s: lam^{T-(s+1)} */
      for (int64_t i = 0; i < dk; ++i) {
        const double ki = w * kb[IDX3(s, i, dk)];
        for (int64_t j = 0; j < dv; ++j) Sb[IDX3(i, j, dv)] += ki * vb[IDX3(s, j, dv)];
      }
    }
  }
}

/* Chunked form in fp64 (self-check of the chunk algebra only).
 * For chunk c holding L tokens (C, or the tail) with local index i = 0..L-1:
 *   O_c[i] = lam^{i+1} S^T q_i + sum_{j<=i} lam^{i-j} (q_i . k_j) v_j
 *   S     <- lam^L S + sum_j lam^{L-1-j} k_j v_j^T
 */
void gla_oracle_fwd_chunked(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                            int64_t C, const double* q, const double* k, const double* v,
                            const double* lam, const double* S0, double* o, double* S_T) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const int64_t h = bh % H;
    const double l = lam[h];
    const double* qb = q + (size_t)bh * T * dk;
    const double* kb = k + (size_t)bh * T * dk;
    const double* vb = v + (size_t)bh * T * dv;
    double* ob = o + (size_t)bh * T * dv;
    double* S = (double*)malloc(sizeof(double) * dk * dv);
    double* Snew = (double*)malloc(sizeof(double) * dk * dv);
    if (S0) memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
    else memset(S, 0, sizeof(double) * dk * dv);
    for (int64_t c0 = 0; c0 < T; c0 += C) {
      const int64_t L = (T - c0 < C) ? (T - c0) : C;
      for (int64_t i = 0; i < L; ++i) {
        const int64_t t = c0 + i;
        const double wr = lam_pow(l, i + 1);
        for (int64_t j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int64_t d = 0; d < dk; ++d) acc += qb[IDX3(t, d, dk)] * S[IDX3(d, j, dv)];
          ob[IDX3(t, j, dv)] = wr * acc;
        }
        for (int64_t jj = 0; jj <= i; ++jj) {
          double qk = 0.0;
          for (int64_t d = 0; d < dk; ++d) qk += qb[IDX3(t, d, dk)] * kb[IDX3(c0 + jj, d, dk)];
          const double w = lam_pow(l, i - jj) * qk;
          for (int64_t j = 0; j < dv; ++j) ob[IDX3(t, j, dv)] += w * vb[IDX3(c0 + jj, j, dv)];
        }
      }
      const double wc = lam_pow(l, L);
      for (int64_t d = 0; d < dk * dv; ++d) Snew[d] = wc * S[d];
      for (int64_t jj = 0; jj < L; ++jj) {
        const double w = lam_pow(l, L - 1 - jj);
        for (int64_t d = 0; d < dk; ++d) {
          const double kd = w * kb[IDX3(c0 + jj, d, dk)];
          for (int64_t j = 0; j < dv; ++j) Snew[IDX3(d, j, dv)] += kd * vb[IDX3(c0 + jj, j, dv)];
        }
      }
      memcpy(S, Snew, sizeof(double) * dk * dv);
    }
    if (S_T) memcpy(S_T + (size_t)bh * dk * dv, S, sizeof(double) * dk * dv);
    free(S);
    free(Snew);
  }
}

/* Backward of the loss  L = sum_t <dO_t, o_t> + <dS_T, S_T>.
 * Forward sweep:  recompute S_t;  dq_t = S_t dO_t.
 * Reverse sweep:  G_T = dS_T + q_T dO_T^T,  G_t = lam G_{t+1} + q_t dO_t^T,
 *                 dk_t = G_t v_t,  dv_t = G_t^T k_t,  dS_0 = lam G_1.
 * dS_T and S0 may be NULL (zero); dS0 may be NULL (not returned). */
void gla_oracle_bwd(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                    const double* q, const double* k, const double* v,
                    const double* lam, const double* S0, const double* dO,
                    const double* dS_T, double* dq, double* dkk, double* dvv, double* dS0) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const int64_t h = bh % H;
    const double l = lam[h];
    const double* qb = q + (size_t)bh * T * dk;
    const double* kb = k + (size_t)bh * T * dk;
    const double* vb = v + (size_t)bh * T * dv;
    const double* gb = dO + (size_t)bh * T * dv;
    double* dqb = dq + (size_t)bh * T * dk;
    double* dkb = dkk + (size_t)bh * T * dk;
    double* dvb = dvv + (size_t)bh * T * dv;
    double* S = (double*)malloc(sizeof(double) * dk * dv);
    /* forward sweep */
    if (S0) memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
    else memset(S, 0, sizeof(double) * dk * dv);
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t i = 0; i < dk; ++i) {
        const double ki = kb[IDX3(t, i, dk)];
        for (int64_t j = 0; j < dv; ++j)
          S[IDX3(i, j, dv)] = l * S[IDX3(i, j, dv)] + ki * vb[IDX3(t, j, dv)];
      }
      for (int64_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) acc += S[IDX3(i, j, dv)] * gb[IDX3(t, j, dv)];
        dqb[IDX3(t, i, dk)] = acc;
      }
    }
    /* reverse sweep; S now holds G */
    if (dS_T) memcpy(S, dS_T + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
    else memset(S, 0, sizeof(double) * dk * dv);
    for (int64_t t = T - 1; t >= 0; --t) {
      const double w = (t == T - 1) ? 1.0 : l; /* G_T = dS_T + q_T dO_T^T */
      for (int64_t i = 0; i < dk; ++i) {
        const double qi = qb[IDX3(t, i, dk)];
        for (int64_t j = 0; j < dv; ++j)
          S[IDX3(i, j, dv)] = w * S[IDX3(i, j, dv)] + qi * gb[IDX3(t, j, dv)];
      }
      for (int64_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) acc += S[IDX3(i, j, dv)] * vb[IDX3(t, j, dv)];
        dkb[IDX3(t, i, dk)] = acc;
      }
      for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < dk; ++i) acc += S[IDX3(i, j, dv)] * kb[IDX3(t, i, dk)];
        dvb[IDX3(t, j, dv)] = acc;
      }
    }
    if (dS0) {
      double* d0 = dS0 + (size_t)bh * dk * dv;
      if (T == 0) {
        if (dS_T) memcpy(d0, dS_T + (size_t)bh * dk * dv, sizeof(double) * dk * dv);
        else memset(d0, 0, sizeof(double) * dk * dv);
      } else {
        for (int64_t i = 0; i < dk * dv; ++i) d0[i] = l * S[i];
      }
    }
    free(S);
  }
}

/* Brute-force backward (self-check of gla_oracle_bwd), 1-indexed t, s:
 *   dq_t  = lam^t S0 dO_t + sum_{s<=t} lam^{t-s} (v_s . dO_t) k_s
 *   dk_s  = sum_{t>=s} lam^{t-s} (v_s . dO_t) q_t + lam^{T-s} dS_T v_s
 *   dv_s  = sum_{t>=s} lam^{t-s} (q_t . k_s) dO_t + lam^{T-s} dS_T^T k_s
 *   dS_0  = sum_t lam^t q_t dO_t^T + lam^T dS_T                              */
void gla_oracle_bwd_bruteforce(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                               const double* q, const double* k, const double* v,
                               const double* lam, const double* S0, const double* dO,
                               const double* dS_T, double* dq, double* dkk, double* dvv,
                               double* dS0) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const int64_t h = bh % H;
    const double l = lam[h];
    const double* qb = q + (size_t)bh * T * dk;
    const double* kb = k + (size_t)bh * T * dk;
    const double* vb = v + (size_t)bh * T * dv;
    const double* gb = dO + (size_t)bh * T * dv;
    const double* S0b = S0 ? S0 + (size_t)bh * dk * dv : NULL;
    const double* dSb = dS_T ? dS_T + (size_t)bh * dk * dv : NULL;
    double* dqb = dq + (size_t)bh * T * dk;
    double* dkb = dkk + (size_t)bh * T * dk;
    double* dvb = dvv + (size_t)bh * T * dv;
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        if (S0b) {
          double sd = 0.0;
          for (int64_t j = 0; j < dv; ++j) sd += S0b[IDX3(i, j, dv)] * gb[IDX3(t, j, dv)];
          acc += lam_pow(l, t + 1) * sd;
        }
        for (int64_t s = 0; s <= t; ++s) {
          double vd = 0.0;
          for (int64_t j = 0; j < dv; ++j) vd += vb[IDX3(s, j, dv)] * gb[IDX3(t, j, dv)];
          acc += lam_pow(l, t - s) * vd * kb[IDX3(s, i, dk)];
        }
        dqb[IDX3(t, i, dk)] = acc;
      }
    }
    for (int64_t s = 0; s < T; ++s) {
      for (int64_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int64_t t = s; t < T; ++t) {
          double vd = 0.0;
          for (int64_t j = 0; j < dv; ++j) vd += vb[IDX3(s, j, dv)] * gb[IDX3(t, j, dv)];
          acc += lam_pow(l, t - s) * vd * qb[IDX3(t, i, dk)];
        }
        if (dSb) {
          double dsv = 0.0;
          for (int64_t j = 0; j < dv; ++j) dsv += dSb[IDX3(i, j, dv)] * vb[IDX3(s, j, dv)];
          acc += lam_pow(l, T - 1 - s) * dsv;
        }
        dkb[IDX3(s, i, dk)] = acc;
      }
      for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t t = s; t < T; ++t) {
          double qk = 0.0;
          for (int64_t i = 0; i < dk; ++i) qk += qb[IDX3(t, i, dk)] * kb[IDX3(s, i, dk)];
          acc += lam_pow(l, t - s) * qk * gb[IDX3(t, j, dv)];
        }
        if (dSb) {
          double dsk = 0.0;
          for (int64_t i = 0; i < dk; ++i) dsk += dSb[IDX3(i, j, dv)] * kb[IDX3(s, i, dk)];
          acc += lam_pow(l, T - 1 - s) * dsk;
        }
        dvb[IDX3(s, j, dv)] = acc;
      }
    }
    if (dS0) {
      double* d0 = dS0 + (size_t)bh * dk * dv;
      for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) {
          double acc = dSb ? lam_pow(l, T) * dSb[IDX3(i, j, dv)] : 0.0;
          for (int64_t t = 0; t < T; ++t)
            acc += lam_pow(l, t + 1) * qb[IDX3(t, i, dk)] * gb[IDX3(t, j, dv)];
          d0[IDX3(i, j, dv)] = acc;
        }
    }
  }
}

/* One recurrent decode step for N sequences x H heads (section "Inference
 * optimization on Trainium2": one new token per step against a fixed-size
 * state):  S <- lam S + k v^T  (in place), then  o = S^T q.
 * q,k [N][H][dk], v,o [N][H][dv], S [N][H][dk][dv]. */
void gla_oracle_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv,
                            const double* q, const double* k, const double* v,
                            const double* lam, double* S, double* o) {
#pragma omp parallel for schedule(static)
  for (int64_t nh = 0; nh < N * H; ++nh) {
    const double l = lam[nh % H];
    const double* qb = q + (size_t)nh * dk;
    const double* kb = k + (size_t)nh * dk;
    const double* vb = v + (size_t)nh * dv;
    double* Sb = S + (size_t)nh * dk * dv;
    double* ob = o + (size_t)nh * dv;
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j)
        Sb[IDX3(i, j, dv)] = l * Sb[IDX3(i, j, dv)] + kb[i] * vb[j];
    for (int64_t j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int64_t i = 0; i < dk; ++i) acc += qb[i] * Sb[IDX3(i, j, dv)];
      ob[j] = acc;
    }
  }
}

int gla_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
