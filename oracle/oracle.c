/*
 * CPU oracle for scaled-dot-product attention and its per-row softmax
 * statistics, in IEEE double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: it is used by the test suite, by the smoke check and by the
 * benchmark's CPU-baseline leg, nowhere else.  It shares no code with the HIP
 * library.
 *
 * What it computes follows "Speed Is All You Need: On-Device Acceleration of
 * Large Diffusion Models via GPU-Aware Optimizations" (Chen et al.), as
 * summarised on the news write-up page (section on improving attention
 * efficiency):
 *   - the partially fused softmax first reduces the logit matrix A to two
 *     numbers per row (an N x 2 tensor), then applies the softmax inside the
 *     product with V;
 *   - the reduction over a row may be cut into blocks whose partial results
 *     are merged into the final pair;
 *   - FlashAttention is exact, so both variants must reach the plain
 *     definition O = softmax(scale * Q K^T) V.
 * The two numbers per row are read as m = max_j a_ij and
 * l = sum_j exp(a_ij - m) (natural base), with the scale inside A.
 *
 * Everything here is the plain definition written out: the full score matrix
 * is materialised, rows are reduced left to right, nothing is blocked, fused
 * or reordered, except in oracle_block_stats, which follows the pages'
 * block-split description on purpose so that it can be checked against the
 * whole-row definition.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>

/* S[i][j] = scale * sum_c q[i][c] * k[j][c]: the logit matrix A. */
void oracle_scores(const double* q, const double* k, int nq, int nk, int d,
                   double scale, double* s) {
  for (int i = 0; i < nq; ++i) {
    for (int j = 0; j < nk; ++j) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += q[(size_t)i * d + c] * k[(size_t)j * d + c];
      s[(size_t)i * nk + j] = scale * acc;
    }
  }
}

/* Row softmax of S with its statistics: m[i] = max_j S[i][j],
 * l[i] = sum_j exp(S[i][j] - m[i]), P[i][j] = exp(S[i][j] - m[i]) / l[i].
 * P may alias S (each row is read completely before it is overwritten). */
void oracle_softmax_rows(const double* s, int nq, int nk, double* p, double* m,
                         double* l) {
  for (int i = 0; i < nq; ++i) {
    const double* row = s + (size_t)i * nk;
    double mx = row[0];
    for (int j = 1; j < nk; ++j)
      if (row[j] > mx) mx = row[j];
    double sum = 0.0;
    for (int j = 0; j < nk; ++j) sum += exp(row[j] - mx);
    for (int j = 0; j < nk; ++j) p[(size_t)i * nk + j] = exp(row[j] - mx) / sum;
    m[i] = mx;
    l[i] = sum;
  }
}

/* O[i][c] = sum_j P[i][j] * v[j][c]. */
void oracle_pv(const double* p, const double* v, int nq, int nk, int d, double* o) {
  for (int i = 0; i < nq; ++i) {
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < nk; ++j) acc += p[(size_t)i * nk + j] * v[(size_t)j * d + c];
      o[(size_t)i * d + c] = acc;
    }
  }
}

/* The pages' block-split reduction of one row of A: the nk entries are cut
 * into consecutive blocks of the given lengths (which sum to nk); each block
 * is reduced to its own (max, sum of exp relative to that max), and the
 * partial pairs are folded left to right with
 *   (m, l) + (m', l') = (M, l exp(m - M) + l' exp(m' - M)),  M = max(m, m').
 * The result equals (max_j a_j, sum_j exp(a_j - max)) up to rounding. */
void oracle_block_stats(const double* row, int nk, const int* block_len, int nblocks,
                        double* m_out, double* l_out) {
  double m = -INFINITY, l = 0.0;
  int start = 0;
  for (int b = 0; b < nblocks; ++b) {
    int len = block_len[b];
    double bm = -INFINITY, bl = 0.0;
    for (int j = start; j < start + len; ++j)
      if (row[j] > bm) bm = row[j];
    for (int j = start; j < start + len; ++j) bl += exp(row[j] - bm);
    if (len > 0) {
      double mm = m > bm ? m : bm;
      l = (l > 0.0 ? l * exp(m - mm) : 0.0) + bl * exp(bm - mm);
      m = mm;
    }
    start += len;
  }
  (void)nk;
  *m_out = m;
  *l_out = l;
}

typedef struct {
  const double *q, *k, *v;
  int nq, nk, d, row0, row1;
  double scale;
  double *s, *o, *ml;
} job_t;

static void* run_rows(void* arg) {
  job_t* j = (job_t*)arg;
  int rows = j->row1 - j->row0;
  if (rows <= 0) return NULL;
  double* s = j->s + (size_t)j->row0 * j->nk;
  double* m = (double*)malloc(sizeof(double) * (size_t)rows);
  double* l = (double*)malloc(sizeof(double) * (size_t)rows);
  oracle_scores(j->q + (size_t)j->row0 * j->d, j->k, rows, j->nk, j->d, j->scale, s);
  oracle_softmax_rows(s, rows, j->nk, s, m, l);
  oracle_pv(s, j->v, rows, j->nk, j->d, j->o + (size_t)j->row0 * j->d);
  if (j->ml) {
    for (int i = 0; i < rows; ++i) {
      j->ml[(size_t)(j->row0 + i) * 2 + 0] = m[i];
      j->ml[(size_t)(j->row0 + i) * 2 + 1] = l[i];
    }
  }
  free(m);
  free(l);
  return NULL;
}

int oracle_attention(const double* q, const double* k, const double* v, int bh,
                     int nq, int nk, int d, double scale, double* o, double* ml,
                     int nthreads) {
  if (bh < 1 || nq < 1 || nk < 1 || d < 1 || !q || !k || !v || !o) return 1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nq) nthreads = nq;
  /* one materialised score matrix per head, shared by the row-split threads */
  double* s = (double*)malloc(sizeof(double) * (size_t)nq * (size_t)nk);
  if (!s) return 2;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)nthreads);
  for (int h = 0; h < bh; ++h) {
    for (int t = 0; t < nthreads; ++t) {
      job_t* j = &jobs[t];
      j->q = q + (size_t)h * nq * d;
      j->k = k + (size_t)h * nk * d;
      j->v = v + (size_t)h * nk * d;
      j->nq = nq;
      j->nk = nk;
      j->d = d;
      j->scale = scale;
      j->row0 = (int)((long long)nq * t / nthreads);
      j->row1 = (int)((long long)nq * (t + 1) / nthreads);
      j->s = s;
      j->o = o + (size_t)h * nq * d;
      j->ml = ml ? ml + (size_t)h * nq * 2 : NULL;
      if (nthreads == 1) run_rows(j);
      else pthread_create(&th[t], NULL, run_rows, j);
    }
    if (nthreads > 1)
      for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  }
  free(jobs);
  free(th);
  free(s);
  return 0;
}
