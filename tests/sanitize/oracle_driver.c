/* Drives every function of the C oracles (oracle/oracle.c, oracle/unet_ops.c)
 * over small and edge-case sizes (one query, one key, head dimension 1,
 * more threads than rows, ragged block splits), so that an AddressSanitizer /
 * UndefinedBehaviorSanitizer build reports any out-of-bounds access, leak or
 * undefined operation.  Exit status 0 when every call returned success and
 * every output is finite. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "oracle.h"
#include "unet_ops.h"

static unsigned long long state = 12345;
static double rnd(void) {
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(state >> 11) * (1.0 / 9007199254740992.0) * 4.0 - 2.0;
}
static double* arr(size_t n) {
  double* p = (double*)malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}
static int finite_all(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int attention_case(int bh, int nq, int nk, int d, int threads) {
  double *q = arr((size_t)bh * nq * d), *k = arr((size_t)bh * nk * d), *v = arr((size_t)bh * nk * d);
  double* o = (double*)malloc(sizeof(double) * (size_t)bh * nq * d);
  double* ml = (double*)malloc(sizeof(double) * (size_t)bh * nq * 2);
  int bad = oracle_attention(q, k, v, bh, nq, nk, d, 1.0 / sqrt((double)d), o, ml, threads) != 0 ||
            !finite_all(o, (size_t)bh * nq * d) || !finite_all(ml, (size_t)bh * nq * 2);
  /* the pieces one by one on the first head */
  double* s = (double*)malloc(sizeof(double) * (size_t)nq * nk);
  double* p = (double*)malloc(sizeof(double) * (size_t)nq * nk);
  double *m = (double*)malloc(sizeof(double) * nq), *l = (double*)malloc(sizeof(double) * nq);
  oracle_scores(q, k, nq, nk, d, 0.5, s);
  oracle_softmax_rows(s, nq, nk, p, m, l);
  oracle_pv(p, v, nq, nk, d, o);
  bad |= !finite_all(o, (size_t)nq * d);
  /* block splits of the first row: one block, single keys, a ragged split */
  int* bl = (int*)malloc(sizeof(int) * nk);
  double bm, bs;
  bl[0] = nk;
  oracle_block_stats(s, nk, bl, 1, &bm, &bs);
  for (int i = 0; i < nk; ++i) bl[i] = 1;
  oracle_block_stats(s, nk, bl, nk, &bm, &bs);
  int nb = 0, left = nk;
  while (left > 0) {
    const int len = left > 3 ? 3 : left;
    bl[nb++] = len;
    left -= len;
  }
  oracle_block_stats(s, nk, bl, nb, &bm, &bs);
  bad |= !isfinite(bm) || !isfinite(bs);
  free(bl); free(s); free(p); free(m); free(l);
  free(q); free(k); free(v); free(o); free(ml);
  return bad;
}

static int unet_case(int n, int c, int hw, int groups, int rows, int f) {
  double *x = arr((size_t)n * c * hw), *g = arr(c), *b = arr(c);
  double* y = (double*)malloc(sizeof(double) * (size_t)n * c * hw);
  double *mean = (double*)malloc(sizeof(double) * (size_t)n * groups), *rstd = (double*)malloc(sizeof(double) * (size_t)n * groups);
  int bad = oracle_group_norm(x, g, b, n, c, hw, groups, 1e-5, y, mean, rstd) != 0 ||
            !finite_all(y, (size_t)n * c * hw);
  bad |= oracle_group_norm(x, NULL, NULL, n, c, hw, groups, 0.0, y, NULL, NULL) != 0;
  bad |= oracle_group_norm(x, g, b, n, c, hw, c + 1, 1e-5, y, NULL, NULL) == 0; /* invalid: must refuse */
  double* h = arr((size_t)rows * 2 * f);
  double* out = (double*)malloc(sizeof(double) * (size_t)rows * f);
  bad |= oracle_geglu(h, rows, f, out) != 0 || !finite_all(out, (size_t)rows * f);
  double gx[5] = {-40.0, -1.0, 0.0, 1.0, 40.0}, gy[5];
  oracle_gelu(gx, 5, gy);
  bad |= !finite_all(gy, 5) || !isfinite(oracle_gelu1(-9.0));
  free(x); free(g); free(b); free(y); free(mean); free(rstd); free(h); free(out);
  return bad;
}

int main(void) {
  int bad = 0;
  const int shapes[][5] = {{1, 1, 1, 1, 1}, {1, 1, 1, 40, 4}, {2, 5, 3, 40, 8}, {1, 17, 33, 80, 3},
                           {3, 64, 1, 160, 2}, {1, 1, 129, 7, 1}, {2, 100, 65, 40, 16}};
  for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
    const int* s = shapes[i];
    if (attention_case(s[0], s[1], s[2], s[3], s[4])) {
      fprintf(stderr, "attention case %zu failed\n", i);
      bad = 1;
    }
  }
  if (unet_case(1, 4, 1, 1, 1, 1) || unet_case(2, 32, 7, 8, 3, 5) || unet_case(1, 64, 33, 32, 17, 64)) {
    fprintf(stderr, "unet ops case failed\n");
    bad = 1;
  }
  printf(bad ? "FAIL\n" : "OK\n");
  return bad;
}
