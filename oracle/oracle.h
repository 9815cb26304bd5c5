/* CPU double-precision oracle for scaled-dot-product attention.
 * Test infrastructure only: see oracle.c.  All matrices are row-major and
 * contiguous; q is [nq][d], k and v are [nk][d], s and p are [nq][nk],
 * o is [nq][d], ml is [nq][2] with (m, l) per row. */
#ifndef ATTN_ORACLE_H
#define ATTN_ORACLE_H
#ifdef __cplusplus
extern "C" {
#endif
void oracle_scores(const double* q, const double* k, int nq, int nk, int d,
                   double scale, double* s);
void oracle_softmax_rows(const double* s, int nq, int nk, double* p, double* m,
                         double* l);
void oracle_pv(const double* p, const double* v, int nq, int nk, int d, double* o);
void oracle_block_stats(const double* row, int nk, const int* block_len, int nblocks,
                        double* m_out, double* l_out);
/* bh heads laid out one after another; returns 0 on success. */
int oracle_attention(const double* q, const double* k, const double* v, int bh,
                     int nq, int nk, int d, double scale, double* o, double* ml,
                     int nthreads);
#ifdef __cplusplus
}
#endif
#endif
