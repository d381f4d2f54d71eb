/*
 * gla_conv_oracle.c -- fp64 CPU oracle of the depthwise causal convolution
 * that feeds the Simple GLA mixer.
 *
 * TEST INFRASTRUCTURE ONLY (same rules as gla_oracle.c: loaded only by the
 * test suite, the package smoke check and the benchmark's CPU-baseline leg;
 * no code shared with the HIP library).
 *
 * Source: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
 * attention model on AWS Trainium2 with native PyTorch", section "i14 and
 * Laplace 3B architecture", paragraph "Normalization and convolution": every
 * channel of the D = 3,072-wide residual stream passes through a causal
 * depthwise Conv1d of width 4 followed by SiLU, giving each position a summary
 * of its last 4 tokens before the mixer; the recurrent state of a sequence
 * holds the convolution window next to the mixer states.
 *
 * Readings (the page gives no formula):
 *   z[t][c] = bias[c] + sum_{j=0..W-1} w[c][j] * x[t - (W-1) + j][c]
 *   y[t][c] = SiLU(z) = z / (1 + exp(-z))
 * so tap W-1 weights the current token.  Inputs before token 0 come from the
 * carried window state_in[W-1][D] (oldest first; zero when absent), and the
 * window after the last token (the last W-1 inputs) is returned for decode.
 * Everything is double precision.  Layouts: x, y [B][T][D]; w [D][W];
 * bias [D]; windows [B][W-1][D].
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* input seen at token s (s may be negative: then it is read from the window) */
static double conv_input(const double* xb, const double* win, int64_t s, int64_t c, int64_t D, int64_t W) {
  if (s >= 0) return xb[(size_t)s * D + c];
  if (!win) return 0.0;
  return win[(size_t)(W - 1 + s) * D + c];
}

void gla_oracle_conv1d(int64_t B, int64_t T, int64_t D, int64_t W, const double* x, const double* w,
                       const double* bias, const double* state_in, double* y, double* state_out) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    const double* xb = x + (size_t)b * T * D;
    const double* win = state_in ? state_in + (size_t)b * (W - 1) * D : NULL;
    double* yb = y + (size_t)b * T * D;
    for (int64_t t = 0; t < T; ++t)
      for (int64_t c = 0; c < D; ++c) {
        double z = bias ? bias[c] : 0.0;
        for (int64_t j = 0; j < W; ++j) z += w[(size_t)c * W + j] * conv_input(xb, win, t - (W - 1) + j, c, D, W);
        yb[(size_t)t * D + c] = silu(z);
      }
    if (state_out)
      for (int64_t j = 0; j < W - 1; ++j)
        for (int64_t c = 0; c < D; ++c)
          state_out[((size_t)b * (W - 1) + j) * D + c] = conv_input(xb, win, T - (W - 1) + j, c, D, W);
  }
}

/* One decode token per sequence: y = SiLU(bias + w . [window, x]); the window
 * then drops its oldest input and appends x (in place). */
void gla_oracle_conv1d_step(int64_t N, int64_t D, int64_t W, const double* x, const double* w,
                            const double* bias, double* state, double* y) {
  for (int64_t n = 0; n < N; ++n) {
    double* win = state + (size_t)n * (W - 1) * D;
    for (int64_t c = 0; c < D; ++c) {
      double z = bias ? bias[c] : 0.0;
      for (int64_t j = 0; j < W - 1; ++j) z += w[(size_t)c * W + j] * win[(size_t)j * D + c];
      z += w[(size_t)c * W + W - 1] * x[(size_t)n * D + c];
      y[(size_t)n * D + c] = silu(z);
      for (int64_t j = 0; j + 1 < W - 1; ++j) win[(size_t)j * D + c] = win[(size_t)(j + 1) * D + c];
      if (W > 1) win[(size_t)(W - 2) * D + c] = x[(size_t)n * D + c];
    }
  }
}
