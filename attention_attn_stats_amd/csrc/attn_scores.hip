// The partially fused softmax over a materialised logit matrix, as the
// write-up draws its data flow: A = scale Q K^T is written to memory by one
// launch, a second launch reduces every row of A to its (m, l) pair with the
// block-split reduction, and a third applies the softmax inside the product
// with V (that one lives in attn_mfma.hip, fwd_kernel<.., kModePVScores>).
//
// Method: "Speed Is All You Need: On-Device Acceleration of Large Diffusion
// Models via GPU-Aware Optimizations" (Chen et al.), news write-up, section on
// improving attention efficiency.
//
// A is stored as float32 (the matrix cores' accumulator type): rounding the
// logits to 16 bits would move exp(a - m) by up to 2^-11 * |a| relative.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef short s8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef int i4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

struct F16 {
  static __device__ __forceinline__ f16v mma32(s8v a, s8v b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
  }
};
struct BF16 {
  static __device__ __forceinline__ f16v mma32(s8v a, s8v b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8v, a), __builtin_bit_cast(b8v, b), c, 0, 0, 0);
  }
};

// Raw buffer resource (stride 0) over `bytes` bytes at p: loads at offsets at
// or past `bytes` return zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// A = scale * Q K^T, float32, [BH][Nq][Nk].  A workgroup of 4 waves computes a
// 128-query x 128-key tile; each wave 32 queries x 128 keys as four 32x32
// tiles on v_mfma_f32_32x32x16 with Q as the A operand (rows = queries) and
// K^T as the B operand, so that lane l ends up holding key l % 32 of 16 query
// rows and every store instruction writes 128 contiguous bytes of a row of A.
// Both operands come straight from memory (16 bytes per lane and K step,
// range-checked buffer loads; dims past d are zero on the Q side).
// ---------------------------------------------------------------------------
constexpr int kSQ = 128, kSK = 128;  // tile of A per workgroup

template <class TR, int D>
__global__ __launch_bounds__(256) void scores_kernel(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k,
                                                     float* __restrict__ a, const Layout lay, int Nq, int Nk,
                                                     int qtiles, int ktiles, float scale) {
  constexpr int KS = (D + 15) / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  int t = blockIdx.x;
  const int kt = t % ktiles;
  t /= ktiles;
  const int qt = t % qtiles;
  const int head = t / qtiles;
  const int q0 = qt * kSQ + wave * 32, k0 = kt * kSK;
  const int qs = lay.q.row, ks_ = lay.k.row;  // row strides (elements)
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(q + head_offset(lay.q, lay.H, head), (uint32_t)((Nq - 1) * qs + D) * 2);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + head_offset(lay.k, lay.H, head), (uint32_t)((Nk - 1) * ks_ + D) * 2);

  // Q fragments: query q0 + l32, dims 16 ks + 8 hi .. +8 (zero past d)
  s8v qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d0 = ks * 16 + hi * 8;
    const i4v x = __builtin_bit_cast(i4v, __builtin_amdgcn_raw_buffer_load_b128(qr, ((q0 + l32) * qs + (d0 < D ? d0 : 0)) * 2, 0, 0));
    qf[ks] = d0 < D ? __builtin_bit_cast(s8v, x) : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
  }
  f16v acc[kSK / 32];
#pragma unroll
  for (int n = 0; n < kSK / 32; ++n) {
    acc[n] = (f16v){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 16 + hi * 8;
      // key k0 + 32 n + l32; past d the Q side is zero, so any finite data will do
      const i4v x = __builtin_bit_cast(i4v, __builtin_amdgcn_raw_buffer_load_b128(kr, ((k0 + 32 * n + l32) * ks_ + (d0 < D ? d0 : 0)) * 2, 0, 0));
      acc[n] = TR::mma32(qf[ks], __builtin_bit_cast(s8v, x), acc[n]);
    }
  }
  float* ah = a + (size_t)head * Nq * Nk;
#pragma unroll
  for (int n = 0; n < kSK / 32; ++n) {
    const int col = k0 + 32 * n + l32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = q0 + (i / 4) * 8 + hi * 4 + (i % 4);
      if (row < Nq && col < Nk) ah[(size_t)row * Nk + col] = acc[n][i] * scale;
    }
  }
}

// ---------------------------------------------------------------------------
// Row statistics of A: (m_i, l_i) for every row, the block-split reduction.
// One wave per row.  The row is cut into blocks of 4 x 16 bytes, one per lane
// and sweep (the 16-byte pieces dealt round robin); a lane reduces each block
// to its (max, sum of exp) pair and merges it into its running pair, and the
// 64 partial pairs are merged with (m,l)+(m',l') = (M, l e^(m-M) +
// l' e^(m'-M)) across the wave -- one launch, nothing but ml written.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void merge(float& m, float& l, float m2, float l2) {
  const float M = __builtin_fmaxf(m, m2);
  // a side that saw no element holds (-inf, 0)
  const float f1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
  const float f2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
  l = l * f1 + l2 * f2;
  m = M;
}

template <bool kVec>  // rows start 16-byte aligned (Nk % 4 == 0): one 16-byte load per block
__global__ __launch_bounds__(256) void rowstats_kernel(const float* __restrict__ a, float* __restrict__ ml,
                                                       long long rows, int Nk) {
  const int lane = threadIdx.x & 63;
  // wave-uniform (and known so to the compiler): the buffer resource of the
  // row lives in scalar registers
  const long long row = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(a + (size_t)row * Nk, (uint32_t)Nk * 4);
  float m = -INFINITY, l = 0.f;  // in exp2 units
  constexpr int U = 4;           // blocks in flight per lane
  for (int c0 = lane * 4; c0 < Nk; c0 += 256 * U) {
    float x[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (kVec) {
        // cast the whole vector: a per-element bit cast of this builtin's
        // result has been compiled into a single-dword load here
        const f4v y = __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(ar, (c0 + 256 * u) * 4, 0, 0));
#pragma unroll
        for (int j = 0; j < 4; ++j) x[u][j] = y[j];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          x[u][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ar, (c0 + 256 * u + j) * 4, 0, 0));
      }
    }
    // this lane's block: its U x 4 elements of this sweep (past Nk: -inf)
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[u][j] = c0 + 256 * u + j < Nk ? x[u][j] * kLog2e : -INFINITY;
        bm = __builtin_fmaxf(bm, x[u][j]);
      }
    float bl = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) bl += __builtin_amdgcn_exp2f(x[u][j] - bm);
    merge(m, l, bm, bl);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const float m2 = __shfl_xor(m, s), l2 = __shfl_xor(l, s);
    merge(m, l, m2, l2);
  }
  if (lane == 0) *(float2*)(ml + row * 2) = make_float2(m / kLog2e, l);
}

template <class TR, int D>
hipError_t launch_scores_t(const Problem& p, float* a) {
  const int qtiles = (p.Nq + kSQ - 1) / kSQ, ktiles = (p.Nk + kSK - 1) / kSK;
  const long long nwg = (long long)p.BH * qtiles * ktiles;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((scores_kernel<TR, D>), dim3((unsigned)nwg), dim3(256), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, a, p.lay, p.Nq, p.Nk, qtiles, ktiles, p.scale);
  return hipGetLastError();
}

template <class TR>
hipError_t scores_by_dim(const Problem& p, float* a) {
  switch (p.d) {
    case 40: return launch_scores_t<TR, 40>(p, a);
    case 80: return launch_scores_t<TR, 80>(p, a);
    case 160: return launch_scores_t<TR, 160>(p, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_scores(const Problem& p, float* a) {
  return p.dt == ATTN_BF16 ? scores_by_dim<BF16>(p, a) : scores_by_dim<F16>(p, a);
}

hipError_t launch_scores_stats(const float* a, float* ml, long long rows, int Nk, hipStream_t stream) {
  const long long nwg = (rows + 3) / 4;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  if ((Nk & 3) == 0)
    hipLaunchKernelGGL(rowstats_kernel<true>, dim3((unsigned)nwg), dim3(256), 0, stream, a, ml, rows, Nk);
  else
    hipLaunchKernelGGL(rowstats_kernel<false>, dim3((unsigned)nwg), dim3(256), 0, stream, a, ml, rows, Nk);
  return hipGetLastError();
}

}  // namespace attn
