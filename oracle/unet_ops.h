/* CPU double-precision oracle for group normalisation and the GELU-gated
 * product.  Test infrastructure only: see unet_ops.c. */
#ifndef ATTN_ORACLE_UNET_OPS_H
#define ATTN_ORACLE_UNET_OPS_H
#include <stddef.h>
#ifdef __cplusplus
extern "C" {
#endif
/* x, y [n][c][hw]; gamma, beta [c] or NULL; mean_out, rstd_out [n][groups] or
 * NULL.  Returns 0, or 1 for invalid sizes (c not a multiple of groups, ...). */
int oracle_group_norm(const double* x, const double* gamma, const double* beta, int n, int c,
                      int hw, int groups, double eps, double* y, double* mean_out,
                      double* rstd_out);
double oracle_gelu1(double x);
void oracle_gelu(const double* x, size_t count, double* y);
/* h [rows][2f] -> out [rows][f]; returns 0, or 1 for invalid sizes. */
int oracle_geglu(const double* h, int rows, int f, double* out);
#ifdef __cplusplus
}
#endif
#endif
