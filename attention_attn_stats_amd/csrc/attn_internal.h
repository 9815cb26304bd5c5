// Internal launch interface between the C ABI (attn_api.cpp) and the kernels.
#ifndef ATTN_INTERNAL_H
#define ATTN_INTERNAL_H

#include <hip/hip_runtime.h>

#include "attn.h"

namespace attn {

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
};

// Matrix-core (fp16 / bf16) kernels.
hipError_t launch_mfma_stats(const Problem& p);
hipError_t launch_mfma_pv(const Problem& p);
hipError_t launch_mfma_flash(const Problem& p);  // writes p.ml when it is non-null

// The partially fused form over a stored logit matrix A (float32).
hipError_t launch_scores(const Problem& p, float* a);                   // A = scale Q K^T
hipError_t launch_scores_stats(const float* a, float* ml, long long rows, int Nk, hipStream_t stream);
hipError_t launch_mfma_pv_scores(const Problem& p);                     // O from p.a, p.ml, p.v

// Vector-ALU float32 kernels.
hipError_t launch_f32_stats(const Problem& p);
hipError_t launch_f32_pv(const Problem& p);
hipError_t launch_f32_flash(const Problem& p);

}  // namespace attn

#endif
