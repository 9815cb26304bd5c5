/*
 * CPU oracle for the two other specialised kernels of the SD UNet, in IEEE
 * double precision: group normalisation and the GELU-gated product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: it is used by the test suite, by the smoke check and by the
 * benchmark's CPU-baseline leg, nowhere else.  It shares no code with the HIP
 * library.
 *
 * What it computes follows "Speed Is All You Need: On-Device Acceleration of
 * Large Diffusion Models via GPU-Aware Optimizations" (Chen et al.), as
 * summarised on the news write-up page (section on the specialised kernels):
 *   - group normalisation splits the channels of a feature map into groups
 *     and normalises every group on its own (one kernel, no intermediate
 *     tensors on the GPU side);
 *   - the GELU activation is evaluated with the Gaussian error function, and
 *     its kernel also takes over the split and the multiplication that come
 *     with it in the UNet (the gated form: one half of a projection times the
 *     GELU of the other half).
 * The pages give neither formula in full; the readings written out here are:
 *   group_norm: per sample n and group g, over the C/G channels of the group
 *     and all H*W positions, mean and biased variance, then
 *     y = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c];
 *   gelu(x) = x * Phi(x) = x / 2 * (1 + erf(x / sqrt 2))  (the exact form,
 *     evaluated through the complementary error function);
 *   geglu: out[r][j] = h[r][j] * gelu(h[r][F + j]) for a row of 2F values
 *     (the first half is the value, the second half the gate).
 * Everything is the plain definition: two passes over a group (mean, then the
 * squared deviations), rows left to right, nothing blocked or fused.
 */
#include "unet_ops.h"

#include <math.h>
#include <stddef.h>

/* x, y: [n][c][hw] (NCHW with H*W flattened); gamma, beta: [c] or NULL
 * (NULL = 1 and 0); mean_out, rstd_out: [n][groups] or NULL. */
int oracle_group_norm(const double* x, const double* gamma, const double* beta, int n, int c,
                      int hw, int groups, double eps, double* y, double* mean_out,
                      double* rstd_out) {
  if (n < 1 || c < 1 || hw < 1 || groups < 1 || c % groups != 0 || !(eps >= 0.0)) return 1;
  const int cg = c / groups;                 /* channels per group */
  const size_t len = (size_t)cg * hw;        /* elements per group */
  for (int s = 0; s < n; ++s) {
    for (int g = 0; g < groups; ++g) {
      /* the group's channels are g*cg .. g*cg + cg - 1: one contiguous span */
      const size_t base = ((size_t)s * c + (size_t)g * cg) * hw;
      double sum = 0.0;
      for (size_t e = 0; e < len; ++e) sum += x[base + e];
      const double mean = sum / (double)len;
      double sq = 0.0;
      for (size_t e = 0; e < len; ++e) {
        const double dev = x[base + e] - mean;
        sq += dev * dev;
      }
      const double var = sq / (double)len;  /* biased: divide by the count */
      const double rstd = 1.0 / sqrt(var + eps);
      for (int ch = 0; ch < cg; ++ch) {
        const int cc = g * cg + ch;
        const double ga = gamma ? gamma[cc] : 1.0;
        const double be = beta ? beta[cc] : 0.0;
        for (int p = 0; p < hw; ++p) {
          const size_t i = base + (size_t)ch * hw + p;
          y[i] = (x[i] - mean) * rstd * ga + be;
        }
      }
      if (mean_out) mean_out[(size_t)s * groups + g] = mean;
      if (rstd_out) rstd_out[(size_t)s * groups + g] = rstd;
    }
  }
  return 0;
}

/* gelu(x) = x * Phi(x), Phi the standard normal distribution function,
 * Phi(x) = (1 + erf(x / sqrt 2)) / 2 = erfc(-x / sqrt 2) / 2; the second form
 * keeps its relative accuracy where Phi is small (x well below zero). */
double oracle_gelu1(double x) { return 0.5 * x * erfc(-x / sqrt(2.0)); }

void oracle_gelu(const double* x, size_t count, double* y) {
  for (size_t i = 0; i < count; ++i) y[i] = oracle_gelu1(x[i]);
}

/* h: [rows][2f], out: [rows][f]; out[r][j] = h[r][j] * gelu(h[r][f + j]). */
int oracle_geglu(const double* h, int rows, int f, double* out) {
  if (rows < 1 || f < 1) return 1;
  for (int r = 0; r < rows; ++r) {
    const double* row = h + (size_t)r * 2 * f;
    for (int j = 0; j < f; ++j) out[(size_t)r * f + j] = row[j] * oracle_gelu1(row[f + j]);
  }
  return 0;
}
