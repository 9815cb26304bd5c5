/*
 * attn.h -- C ABI of the MI355X (gfx950) attention library libattn.so.
 *
 * The library computes scaled-dot-product attention
 *     O = softmax(scale * Q K^T) V          (softmax over the key axis)
 * in the two forms described in "Speed Is All You Need: On-Device
 * Acceleration of Large Diffusion Models via GPU-Aware Optimizations"
 * (Chen et al.), news write-up, section on improving attention efficiency:
 *
 *  - partially fused softmax: one pass reduces every row of the logit matrix
 *    A = scale * Q K^T to an (m, l) pair -- an N x 2 tensor -- with the row
 *    cut into key blocks whose partial pairs are merged inside the same
 *    launch; a second pass applies the softmax inside the product with V, so
 *    softmax(A) is never stored (attn_stats + attn_pv);
 *  - FlashAttention: one tiled launch that reads Q, K, V once and keeps the
 *    running softmax state on chip; it is exact, so it reaches the same O
 *    (attn_flash);
 *  - the same write-up picks between the two per GPU and head dimension; here
 *    the choice is made by timing both on the device (attn_select, and
 *    attn_forward with ATTN_AUTO).
 *
 * Further below: the partially fused form over a stored logit matrix
 * (attn_scores*, the write-up's literal data flow), the four operations on
 * strided tensors (attn_*_strided), and the UNet's two other specialised
 * kernels of the same write-up (attn_group_norm, attn_geglu).
 *
 * Definitions used throughout (the pages name the two per-row quantities
 * only as "L and S"; they are read here as the row maximum and the row sum
 * of exponentials relative to it, in natural-log units, scale included):
 *     a_ij = scale * sum_c q_ic k_jc
 *     m_i  = max_j a_ij
 *     l_i  = sum_j exp(a_ij - m_i)          (so 1 <= l_i <= Nk)
 *     O_ic = sum_j exp(a_ij - m_i) v_jc / l_i
 *
 * Layouts of the functions without "_strided" (dense, row-major):
 *     q, out : [B][H][Nq][d]   element type given by `dt`
 *     k, v   : [B][H][Nk][d]   element type given by `dt`
 *     ml     : [B][H][Nq][2]   float32, ml[..][0] = m, ml[..][1] = l
 * All pointers are DEVICE pointers on the current HIP device.  The caller owns
 * every buffer; the library allocates nothing on these paths, never frees
 * caller memory and does not synchronise (attn_select and the first
 * ATTN_AUTO call for a new shape are the exceptions, see below).  Work is
 * enqueued on `stream` (a hipStream_t passed as void*, NULL = default stream)
 * and is complete when that stream is; buffers must stay valid until then.
 *
 * Supported: d in {40, 80, 160}; dt in {ATTN_F32, ATTN_F16, ATTN_BF16};
 * any B, H, Nq, Nk >= 1 with B*H*max(Nq,Nk)*d < 2^31 elements per tensor;
 * scale finite and > 0 (the usual 1/sqrt(d) softmax temperature).  q, k, v,
 * out must be 16-byte aligned and ml 8-byte aligned.  out may be q itself (each
 * query row is read before its output row is written, by the same workgroup)
 * but must not share memory with k or v, which every workgroup of a head reads.
 * F16/BF16 run on the matrix cores with float32 accumulation and float32
 * softmax state; F32 is a vector-ALU float32 path kept for exactness checks.
 *
 * Errors: arguments are validated before anything is launched; on an error
 * nothing is written.  A launch failure reported by the HIP runtime is
 * returned as ATTN_ERR_HIP (outputs are then unspecified).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h> /* size_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null required pointer, pointer not 16-byte
                               aligned (ml: 8-byte), dimension < 1, scale not
                               finite and > 0, tensor of 2^31 or more elements */
  ATTN_ERR_UNSUPPORTED = 2, /* d not in {40, 80, 160}, unknown dtype/variant */
  ATTN_ERR_HIP = 3,         /* the HIP runtime reported an error */
  ATTN_STATUS_INT_ = 0x7fffffff
} attn_status;

/* (The *_INT_ members are not values: they give each enumeration the range of
 * int, so that an out-of-range value passed by a caller is an argument the
 * library refuses, not undefined behaviour in the C++ implementation.) */
typedef enum { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2, ATTN_DTYPE_INT_ = 0x7fffffff } attn_dtype;

typedef enum {
  ATTN_AUTO = 0,          /* pick by measurement, cached per shape */
  ATTN_PARTIAL_FUSED = 1, /* attn_stats then attn_pv */
  ATTN_FLASH = 2,         /* attn_flash */
  ATTN_VARIANT_INT_ = 0x7fffffff
} attn_variant;

/* Partially fused softmax, pass 1: per-row statistics of A = scale * Q K^T.
 * Writes ml[b][h][i] = (m_i, l_i).  Each row's key range is cut into blocks;
 * every block is reduced to its own (max, sum of exp) and the partial pairs
 * are merged with (m,l)+(m',l') = (M, l e^(m-M) + l' e^(m'-M)), M = max(m,m'),
 * all inside this single launch (write-up, attention section: the block-split
 * reduction that raises the parallelism of the A -> (L, S) mapping).
 * A is recomputed from Q and K, never read from or written to memory.
 * q: [B][H][Nq][d], k: [B][H][Nk][d] (dt); ml: [B][H][Nq][2] float32, written. */
attn_status attn_stats(const void* q, const void* k, float* ml, int B, int H, int Nq,
                       int Nk, int d, float scale, attn_dtype dt, void* stream);

/* Partially fused softmax, pass 2: O = softmax(A) V using the statistics from
 * attn_stats, with the exponentials, the normalisation and the product with V
 * fused in one launch (write-up, attention section).
 * ml: [B][H][Nq][2] float32 as written by attn_stats (read only);
 * out: [B][H][Nq][d] (dt), written. */
attn_status attn_pv(const void* q, const void* k, const void* v, const float* ml, void* out,
                    int B, int H, int Nq, int Nk, int d, float scale, attn_dtype dt,
                    void* stream);

/* FlashAttention forward: one launch, tiled over keys with the online
 * (running max / running sum) softmax, exact up to rounding (write-up,
 * attention section).  ml_out may be NULL; if given, the final (m, l) of every
 * row is written in the same convention as attn_stats.  With dt = ATTN_F16,
 * d = 40, more than 1024 keys (any key count when the environment sets
 * ATTN_FA40=1; none with ATTN_FA40=0) and ml_out NULL, the scores are formed from q
 * scaled by scale * log2(e) and rounded to fp16 (a relative 2^-11 per product
 * term on top of the float32 accumulation); rows whose first 32 keys put the
 * reference beyond +-64 (exp2 units) are recomputed with the scale in float32. */
attn_status attn_flash(const void* q, const void* k, const void* v, void* out, float* ml_out,
                       int B, int H, int Nq, int Nk, int d, float scale, attn_dtype dt,
                       void* stream);

/* Full forward: computes `out`.  ATTN_PARTIAL_FUSED runs attn_stats then
 * attn_pv (two launches) and needs `ml` (it then holds the statistics);
 * ATTN_FLASH runs attn_flash without statistics output, `ml` is not touched
 * (call attn_flash with ml_out to get them); ATTN_AUTO uses the cached choice for this
 * shape, and on the first call for a shape times both variants on the
 * caller's buffers (synchronising `stream` once) before caching the winner
 * (if `ml` is NULL only FLASH is eligible); on a stream being captured into
 * a graph, or when `out` shares memory with q, k or v (in place over q, say),
 * a shape not yet timed takes attn_default_variant(d) instead, uncached, as
 * nothing may synchronise in a capture and repeated runs would read their
 * own output.  The environment variable
 * ATTN_VARIANT=pf|flash overrides ATTN_AUTO. */
attn_status attn_forward(const void* q, const void* k, const void* v, void* out, float* ml,
                         int B, int H, int Nq, int Nk, int d, float scale, attn_variant var,
                         attn_dtype dt, void* stream);

/* ---- Strided tensors -----------------------------------------------------
 * The same four operations on q, k, v, out laid out with arbitrary element
 * strides, e.g. the [B][N][H*d] activations of a UNet attention block viewed
 * as [B][H][N][d] without a transpose (batch = N*H*d, head = d, row = H*d).
 * Element (b, h, n, c) of a tensor is at b*batch + h*head + n*row + c; the d
 * elements of a row are contiguous.  Requirements per tensor: strides >= 0,
 * d <= row <= 2^20, all three strides multiples of 16 bytes (8 elements for
 * F16/BF16, 4 for F32), one head's rows within 2^30 elements and the whole
 * tensor within 2^31.  Strides of 0 share data (e.g. one k and v for every
 * batch element) and are allowed for the inputs; out must overlap neither
 * itself nor the inputs.  ml stays dense [B][H][Nq][2].  A NULL layout is the
 * dense layout: each function above is its *_strided form with NULL.
 * Violations return ATTN_ERR_INVALID_ARG before anything is launched. */
typedef struct {
  long long batch, head, row; /* element strides */
} attn_strides;
typedef struct {
  attn_strides q, k, v, out; /* v and out are ignored where not used */
} attn_layout;

attn_status attn_stats_strided(const void* q, const void* k, float* ml, const attn_layout* layout, int B,
                               int H, int Nq, int Nk, int d, float scale, attn_dtype dt, void* stream);
attn_status attn_pv_strided(const void* q, const void* k, const void* v, const float* ml, void* out,
                            const attn_layout* layout, int B, int H, int Nq, int Nk, int d, float scale,
                            attn_dtype dt, void* stream);
attn_status attn_flash_strided(const void* q, const void* k, const void* v, void* out, float* ml_out,
                               const attn_layout* layout, int B, int H, int Nq, int Nk, int d, float scale,
                               attn_dtype dt, void* stream);
attn_status attn_forward_strided(const void* q, const void* k, const void* v, void* out, float* ml,
                                 const attn_layout* layout, int B, int H, int Nq, int Nk, int d, float scale,
                                 attn_variant var, attn_dtype dt, void* stream);

/* ---- The partially fused softmax over a stored logit matrix ------------
 * The same two passes with A = scale * Q K^T written to memory first, as the
 * write-up draws the data flow (A is the input of the statistics pass and of
 * the softmax-times-V pass).  The fused entry points above recompute A on
 * chip instead; these three exist to run the pages' literal data flow and to
 * measure what storing A costs.  Layout of A: [B][H][Nq][Nk] float32 (the
 * accumulator type: 16-bit logits would move exp(a - m) by up to 2^-11 |a|).
 * Limits in addition to the ones above: Nq * Nk * 4 < 2^31 (one head's A),
 * a 4-byte aligned; F16 and BF16 only (F32 returns ATTN_ERR_UNSUPPORTED). */

/* A = scale * Q K^T for every head.  q: [B][H][Nq][d], k: [B][H][Nk][d] (dt);
 * a: [B][H][Nq][Nk] float32, written. */
attn_status attn_scores(const void* q, const void* k, float* a, int B, int H, int Nq, int Nk, int d,
                        float scale, attn_dtype dt, void* stream);

/* The block-split reduction of every row of a stored A to (m, l), one launch
 * (write-up, attention section): each row is cut into 16-byte blocks, every
 * block reduced to its own (max, sum of exp) pair, the pairs merged with the
 * rule given for attn_stats.  a: [B][H][Nq][Nk] float32 (read only);
 * ml: [B][H][Nq][2] float32, written. */
attn_status attn_scores_stats(const float* a, float* ml, int B, int H, int Nq, int Nk, void* stream);

/* O = softmax(A) V from a stored A and its statistics, exponentials,
 * normalisation and the product with V fused in one launch.  a, ml as above
 * (read only); v: [B][H][Nk][d], out: [B][H][Nq][d] (dt), written. */
attn_status attn_scores_pv(const float* a, const float* ml, const void* v, void* out, int B, int H, int Nq,
                           int Nk, int d, attn_dtype dt, void* stream);

/* ---- The two other specialised kernels of the UNet ------------------------
 * "Speed Is All You Need" (Chen et al.), news write-up, section on the
 * specialised kernels: group normalisation as one GPU command with no
 * intermediate tensor, and GELU evaluated with the error function in one pass
 * together with the split and the multiplication around it. */

/* Group normalisation of x [N][C][HW] (NCHW, spatial dims flattened) with G
 * groups of C/G consecutive channels: per (n, g) the mean and the biased
 * variance over the group's (C/G)*HW elements, then
 * y = (x - mean) / sqrt(var + eps) * gamma[c] + beta[c].  Statistics in
 * float32 (pairwise merged moments, never sums of squares), deterministic.
 * gamma, beta: [C] in dt, or NULL for 1 and 0.  y [N][C][HW] in dt, written;
 * y may equal x.  When a group fits one workgroup's registers (up to 131072
 * fp16/bf16 or 65536 fp32 elements when x, y are 16-byte aligned and HW*size
 * is a multiple of 16 bytes; 16384 elements otherwise) and the groups fill
 * the chip or are small, it is normalised in one launch, x read once, with
 * no intermediate tensor.  Otherwise the groups are split over several
 * workgroups -- in one launch when they can all be resident, else in two --
 * with a workspace of attn_group_norm_workspace_size() bytes (device memory,
 * 8-byte aligned, zero-filled before its first use; the kernels leave it
 * ready for the next call of any shape; calls sharing one workspace must not
 * overlap in time); workspace may be NULL when that size is 0.  A call on a
 * stream that is being captured into a graph, or in place (y == x), takes the
 * two-launch form instead of the one-launch split: the latter tells a call's
 * data in the workspace from an earlier call's by a tag chosen on the host
 * at launch, which every replay of a graph would repeat, and its bounded
 * wait falls back to reading its partners' slices of x.
 * Requirements: sizes >= 1, C a multiple of G, eps finite and >= 0, pointers
 * aligned to the element size, (C/G)*HW < 2^31, N*C*HW < 2^40; else
 * ATTN_ERR_INVALID_ARG before anything is launched (also for a missing or
 * short workspace). */
attn_status attn_group_norm(const void* x, const void* gamma, const void* beta, void* y, void* workspace,
                            size_t workspace_bytes, int N, int C, int HW, int G, float eps, attn_dtype dt,
                            void* stream);

/* attn_group_norm for callers that cannot allocate device memory (code
 * under graph capture, serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels, with the workspace taken from a fixed array
 * of 262144 bytes that the library holds on each device until the process
 * ends (the first call on a device looks its address up; nothing is
 * allocated or freed).  Every call on a device shares that device's array,
 * so calls that overlap in time on one device (different streams, threads
 * or processes) race and must not be issued.  A problem whose workspace
 * (attn_group_norm_workspace_size) exceeds 262144 bytes returns
 * ATTN_ERR_INVALID_ARG before anything is launched; other requirements and
 * errors as attn_group_norm. */
attn_status attn_group_norm_static(const void* x, const void* gamma, const void* beta, void* y, int N, int C,
                                   int HW, int G, float eps, attn_dtype dt, void* stream);

/* Workspace bytes attn_group_norm needs for this problem (0: none), for a
 * call on any stream, captured or not.  The alignment of x and y enters the
 * plan, so pass the pointers that will be used.  Returns 0 for invalid
 * arguments as well. */
size_t attn_group_norm_workspace_size(const void* x, const void* y, int N, int C, int HW, int G,
                                      attn_dtype dt);

/* GELU-gated product: h [rows][2F] -> out [rows][F],
 * out[r][j] = h[r][j] * gelu(h[r][F + j]), gelu(g) = g Phi(g) =
 * g (1 + erf(g / sqrt 2)) / 2 (the exact form), float32 arithmetic.  The
 * first half of a row is the value, the second half the gate.  h read only,
 * out written (must not overlap h).  Requirements: rows, F >= 1,
 * rows*F < 2^31 - 2^9, pointers aligned to the element size; else
 * ATTN_ERR_INVALID_ARG. */
attn_status attn_geglu(const void* h, void* out, int rows, int F, attn_dtype dt, void* stream);

/* The variant ATTN_AUTO uses for this shape.  On a cache miss it allocates
 * temporary device buffers, fills q, k and v with seeded stand-in values
 * (uniform, zero mean, unit variance: non-zero data like the activations it
 * stands for), times both variants on `stream`, frees the buffers and caches
 * the winner, so it synchronises and may allocate; call it outside timed
 * regions.  (attn_forward with ATTN_AUTO times a cache miss on the caller's
 * own buffers instead.)  On a stream being captured into a graph a cache
 * miss returns attn_default_variant(d) without timing or caching.  Returns
 * ATTN_AUTO (0) on error. */
attn_variant attn_select(int B, int H, int Nq, int Nk, int d, attn_dtype dt, void* stream);

/* Before any measurement the choice follows the write-up's own rule: the
 * fused single pass for head dimension 40, the two-pass form otherwise. */
attn_variant attn_default_variant(int d);

/* Forget all cached ATTN_AUTO decisions (thread-safe). */
void attn_select_reset(void);

/* Static text for a status code. */
const char* attn_status_string(attn_status s);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H */
