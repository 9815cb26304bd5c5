// Internal launch interface between the C ABI (attn_api.cpp) and the kernels.
#ifndef ATTN_INTERNAL_H
#define ATTN_INTERNAL_H

#include <hip/hip_runtime.h>

#include "attn.h"

namespace attn {

// Element strides of a [B][H][N][d] tensor whose d elements are contiguous:
// element (b, h, n, c) sits at b * batch + h * head + n * row + c.
struct Strides {
  long long batch, head;
  int row;
};
// The four tensors' strides and the head count that splits a batch-major head
// index bh into (bh / H, bh % H).
struct Layout {
  Strides q, k, v, o;
  int H;
};
// Offset of head bh's first row.
__host__ __device__ inline long long head_offset(const Strides& s, int H, int bh) {
  return (long long)(bh / H) * s.batch + (long long)(bh % H) * s.head;
}
inline Strides dense_strides(int N, int d, int H) {
  Strides s;
  s.batch = (long long)H * N * d;
  s.head = (long long)N * d;
  s.row = d;
  return s;
}

// One problem: BH independent heads of [Nq x d] queries against [Nk x d]
// keys/values, all pointers device pointers, validated by the caller.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* ml;
  const float* a;  // stored logits [BH][Nq][Nk] float32 (the *_scores entry points), else null
  int BH, Nq, Nk, d;
  float scale;
  attn_dtype dt;
  hipStream_t stream;
  Layout lay;  // strides of q, k, v, out (ml and a are always dense)
};

// Matrix-core (fp16 / bf16) kernels.
hipError_t launch_mfma_stats(const Problem& p);
hipError_t launch_mfma_pv(const Problem& p);
hipError_t launch_mfma_flash(const Problem& p);  // writes p.ml when it is non-null
// The software-pipelined head-dimension-40 kernels (fp16 / bf16, dense or
// strided); `cus` = compute units of the device.
hipError_t launch_fa40_flash(const Problem& p, int cus);  // writes p.ml when it is non-null
hipError_t launch_fa40_pv(const Problem& p, int cus);
// The short-key-range single pass (attn_short.hip): every key of a head in
// one block per wave, for Nk <= short_max_keys(d) (0 for unsupported d).
int short_max_keys(int d);
hipError_t launch_short_flash(const Problem& p, int cus);  // writes p.ml when it is non-null

// The partially fused form over a stored logit matrix A (float32).
hipError_t launch_scores(const Problem& p, float* a);                   // A = scale Q K^T
hipError_t launch_scores_stats(const float* a, float* ml, long long rows, int Nk, hipStream_t stream);
hipError_t launch_mfma_pv_scores(const Problem& p);                     // O from p.a, p.ml, p.v

// Seeded stand-in values (uniform, zero mean, unit variance) for n elements
// of type dt at p: the data the variant selector times a shape on.
hipError_t launch_fill_uniform(void* p, size_t n, attn_dtype dt, unsigned seed, hipStream_t stream);

// Group normalisation of x [N][C][HW] (y may equal x).  The workspace is
// needed only by groups too large for one workgroup's registers.
struct GroupNormProblem {
  const void* x;
  const void* gamma;
  const void* beta;
  void* y;
  void* workspace;
  size_t workspace_bytes;
  int N, C, HW, G;
  float eps;
  attn_dtype dt;
  hipStream_t stream;
};
size_t group_norm_workspace(const GroupNormProblem& p);  // bytes the launch plan needs (0: none)
hipError_t launch_group_norm(const GroupNormProblem& p);
// The allocation-free form's fixed per-device workspace (a static device
// array of kGnStaticScratchBytes): its device address on the current device.
constexpr size_t kGnStaticScratchBytes = 256 * 1024;  // 16384 slices of tagged moments
hipError_t group_norm_static_scratch(void** ptr);

// GELU-gated product: h [rows][2F] -> out [rows][F].
struct GegluProblem {
  const void* h;
  void* out;
  int rows, F;
  attn_dtype dt;
  hipStream_t stream;
};
hipError_t launch_geglu(const GegluProblem& p);

// Vector-ALU float32 kernels.
hipError_t launch_f32_stats(const Problem& p);
hipError_t launch_f32_pv(const Problem& p);
hipError_t launch_f32_flash(const Problem& p);

}  // namespace attn

#endif
