// Vector-ALU float32 attention kernels (the ATTN_F32 element type).
//
// These serve callers that need float32 end to end and are the path held to
// the tight float32 tolerance.  Same three operations as the matrix-core
// kernels ("Speed Is All You Need", Chen et al., news write-up, section on
// improving attention efficiency): the row statistics (m, l) of
// A = scale Q K^T with a block-split reduction, the fused softmax-times-V pass
// that consumes them, and the single-pass online-softmax (FlashAttention)
// forward.
//
// One wave per query row, four rows per workgroup.  For the statistics every
// lane reduces its own subset of keys (keys lane, lane+64, ...) to a
// (max, sum of exp) pair -- the blocks of the block-split reduction -- and the
// 64 partial pairs are merged with the (m, l) merge rule across the wave.
// The product with V walks the keys in chunks of 64: each lane computes one
// weight, the weights go through LDS, and the lanes switch to the d output
// columns (lane, lane+64, lane+128) for the accumulation.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kRows = 4;  // query rows (= waves) per workgroup
constexpr int kMaxD = 160;

struct Pair {
  float m, l;
};

// (m, l) + (m', l') = (M, l e^(m - M) + l' e^(m' - M)); (-inf, 0) is the identity
__device__ __forceinline__ Pair merge(Pair a, Pair b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return Pair{-INFINITY, 0.f};
  return Pair{M, a.l * expf(a.m - M) + b.l * expf(b.m - M)};
}

__device__ __forceinline__ Pair wave_merge(Pair p) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Pair o{__shfl_xor(p.m, off), __shfl_xor(p.l, off)};
    p = merge(p, o);
  }
  return p;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// a = scale * q . k for one key
__device__ __forceinline__ float logit(const float* qs, const float* kp, int D, float scale) {
  float acc = 0.f;
  for (int c = 0; c < D; ++c) acc = fmaf(qs[c], kp[c], acc);
  return scale * acc;
}

constexpr int kStats = 0, kPV = 1, kFlash = 2;

template <int MODE>
__global__ __launch_bounds__(64 * kRows) void f32_kernel(const float* __restrict__ q,
                                                         const float* __restrict__ k,
                                                         const float* __restrict__ v,
                                                         float* __restrict__ out,
                                                         float* __restrict__ ml, const Layout lay,
                                                         int BH, int Nq, int Nk, int D, float scale) {
  __shared__ float qs[kRows][kMaxD];
  __shared__ float ps[kRows][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long grow = (long long)blockIdx.x * kRows + wave;  // global row over all heads
  const bool live = grow < (long long)BH * Nq;
  const int head = live ? (int)(grow / Nq) : 0;
  const int row = live ? (int)(grow - (long long)head * Nq) : 0;
  const float* kh = k + head_offset(lay.k, lay.H, head);
  const float* vh = MODE == kStats ? nullptr : v + head_offset(lay.v, lay.H, head);
  const int kr = lay.k.row, vr_ = lay.v.row;
  const float* qp = q + head_offset(lay.q, lay.H, head) + (size_t)row * lay.q.row;
  for (int c = lane; c < D; c += 64) qs[wave][c] = live ? qp[c] : 0.f;
  __syncthreads();

  if constexpr (MODE == kStats) {
    Pair p{-INFINITY, 0.f};
    for (int j = lane; j < Nk; j += 64) {
      const float a = logit(qs[wave], kh + (size_t)j * kr, D, scale);
      p = merge(p, Pair{a, 1.f});
    }
    p = wave_merge(p);
    if (live && lane == 0) *(float2*)(ml + ((size_t)head * Nq + row) * 2) = make_float2(p.m, p.l);
    return;
  } else {
    float acc[3] = {0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    if constexpr (MODE == kPV) {
      if (live) {
        const float2 st = *(const float2*)(ml + ((size_t)head * Nq + row) * 2);
        m = st.x;
        l = st.y;
      }
    }
    for (int j0 = 0; j0 < Nk; j0 += 64) {
      const int j = j0 + lane;
      const float a = j < Nk ? logit(qs[wave], kh + (size_t)j * kr, D, scale) : -INFINITY;
      float pj;
      if constexpr (MODE == kFlash) {
        const float mn = fmaxf(m, wave_max(a));  // finite: every chunk holds a key
        const float alpha = expf(m - mn);
        pj = expf(a - mn);
        l = l * alpha + wave_sum(pj);
#pragma unroll
        for (int t = 0; t < 3; ++t) acc[t] *= alpha;
        m = mn;
      } else {
        pj = expf(a - m);
      }
      ps[wave][lane] = pj;
      __syncthreads();
      const int nj = min(64, Nk - j0);
      for (int jj = 0; jj < nj; ++jj) {
        const float w = ps[wave][jj];
        const float* vr = vh + (size_t)(j0 + jj) * vr_;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const int c = lane + 64 * t;
          if (c < D) acc[t] = fmaf(w, vr[c], acc[t]);
        }
      }
      __syncthreads();
    }
    if (live) {
      const float inv = 1.f / l;
      float* op = out + head_offset(lay.o, lay.H, head) + (size_t)row * lay.o.row;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int c = lane + 64 * t;
        if (c < D) op[c] = acc[t] * inv;
      }
      if constexpr (MODE == kFlash) {
        if (ml && lane == 0) *(float2*)(ml + ((size_t)head * Nq + row) * 2) = make_float2(m, l);
      }
    }
  }
}

template <int MODE>
hipError_t launch(const Problem& p) {
  const long long rows = (long long)p.BH * p.Nq;
  const long long blocks = (rows + kRows - 1) / kRows;
  if (blocks > 0x7fffffffLL || p.d > kMaxD) return hipErrorInvalidValue;
  hipLaunchKernelGGL((f32_kernel<MODE>), dim3((unsigned)blocks), dim3(64 * kRows), 0, p.stream,
                     (const float*)p.q, (const float*)p.k, (const float*)p.v, (float*)p.out, p.ml,
                     p.lay, p.BH, p.Nq, p.Nk, p.d, p.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_f32_stats(const Problem& p) { return launch<kStats>(p); }
hipError_t launch_f32_pv(const Problem& p) { return launch<kPV>(p); }
hipError_t launch_f32_flash(const Problem& p) { return launch<kFlash>(p); }

}  // namespace attn
