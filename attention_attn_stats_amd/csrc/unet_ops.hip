// The two other specialised kernels of the SD UNet: group normalisation in one
// launch with no intermediate tensor, and the GELU-gated product (the split
// of a projection into value and gate, GELU of the gate, and the product) in
// one pass.
//
// Method: "Speed Is All You Need: On-Device Acceleration of Large Diffusion
// Models via GPU-Aware Optimizations" (Chen et al.), news write-up, section on
// the specialised kernels.  The pages name the operations only; the formulas
// taken are group statistics over the C/G consecutive channels of a group and
// all spatial positions (biased variance, eps inside the square root, then a
// per-channel affine), gelu(g) = g Phi(g) with the error function, and
// out = value * gelu(gate) with the value in the first half of a row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "attn_internal.h"

namespace attn {
namespace {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

// Element types: VW elements per 16-byte vector, conversions through float.
struct EF16 {
  static constexpr int VW = 8;
  static __device__ __forceinline__ void unpack(uint4 u, float* f) {
    const h8v v = __builtin_bit_cast(h8v, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    h8v v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (_Float16)f[i];
    return __builtin_bit_cast(uint4, v);
  }
  static __device__ __forceinline__ float get(const void* p, size_t i) { return (float)((const _Float16*)p)[i]; }
  static __device__ __forceinline__ void put(void* p, size_t i, float f) { ((_Float16*)p)[i] = (_Float16)f; }
};
struct EBF16 {
  static constexpr int VW = 8;
  static __device__ __forceinline__ void unpack(uint4 u, float* f) {
    const b8v v = __builtin_bit_cast(b8v, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    b8v v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)f[i];  // round to nearest even
    return __builtin_bit_cast(uint4, v);
  }
  static __device__ __forceinline__ float get(const void* p, size_t i) { return (float)((const __bf16*)p)[i]; }
  static __device__ __forceinline__ void put(void* p, size_t i, float f) { ((__bf16*)p)[i] = (__bf16)f; }
};
struct EF32 {
  static constexpr int VW = 4;
  static __device__ __forceinline__ void unpack(uint4 u, float* f) {
    const f4v v = __builtin_bit_cast(f4v, u);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = v[i];
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    const f4v v = {f[0], f[1], f[2], f[3]};
    return __builtin_bit_cast(uint4, v);
  }
  static __device__ __forceinline__ float get(const void* p, size_t i) { return ((const float*)p)[i]; }
  static __device__ __forceinline__ void put(void* p, size_t i, float f) { ((float*)p)[i] = f; }
};

// ---------------------------------------------------------------------------
// Group normalisation.  x, y: [N][C][HW], so group (n, g) is one contiguous
// span of L = (C/G) HW elements, cut into 16-byte vectors of VW elements
// (HW a multiple of VW keeps every vector inside one channel).
//
// Moments (count, mean, M2 = sum of squared deviations) are reduced per
// thread with two passes over the thread's own values, then merged pairwise,
// (n, m, M2) + (n', m', M2') = (n + n', m + d n'/(n + n'),
// M2 + M2' + d^2 n n'/(n + n')), d = m' - m, in a fixed order, so results are
// deterministic and never rely on E[x^2] - E[x]^2.
//
// Three forms, all reading x from HBM once except the last:
//  - gn_fused_kernel: one 1024-thread workgroup per group holds the group in
//    registers (up to 16 vectors per thread: 131072 fp16/bf16 or 65536 fp32
//    elements), issues every load before using any, merges the moments
//    across the workgroup and writes the group from registers.  Used when
//    the groups fill the chip or are small.
//  - gn_coop_kernel: S workgroups per group, each holding its slice in
//    registers, exchange slice moments through a small workspace as words
//    tagged with the call's epoch (bounded wait, see there) -- one launch for
//    the few large groups of a batch-2 UNet; not used on a stream being
//    captured into a graph, whose replays would repeat the epoch.
//  - gn_partial_kernel + gn_apply_kernel: two launches over S slices (the
//    first writes each slice's moments, the second merges its group's
//    moments in slice order and normalises its slice, reading x again), for
//    groups beyond what the resident workgroups can hold.
// ---------------------------------------------------------------------------
constexpr int kGnFusedThreads = 1024, kGnMaxRv = 16;
constexpr int kGnSliceThreads = 256, kGnSliceBatch = 4;  // vectors in flight per thread when streaming
constexpr long long kGnSliceTarget = 512;                  // workgroups the two-launch path aims for
constexpr long long kGnFusedMinGroups = 256;               // groups that fill the chip in one launch

struct GnArgs {
  const void* x;
  const void* gamma;  // [C] or null
  const void* beta;   // [C] or null
  void* y;
  // [groups][S][2] slice moments (split forms) as 64-bit words: the float
  // bits of the mean (word 0) or of M2 (word 1) in the low half, the call's
  // epoch in the high half
  unsigned long long* ws;
  unsigned epoch;      // nonzero, different for every call on a workspace
  int spin_limit;      // polls before a workgroup stops waiting for its group
  long long L;         // elements per group
  long long slice_vec; // vectors per slice (the last slice of a group may be shorter)
  int HW, G, Cg, S;
  float eps;
};

struct Moments {
  float n, mean, m2;
};

__device__ __forceinline__ unsigned long long tag(float v, unsigned epoch) {
  return ((unsigned long long)epoch << 32) | __float_as_uint(v);
}
__device__ __forceinline__ float untag(unsigned long long w) { return __uint_as_float((unsigned)w); }

__device__ __forceinline__ void merge(Moments& a, const Moments& b) {
  if (b.n == 0.f) return;
  if (a.n == 0.f) {
    a = b;
    return;
  }
  const float n = a.n + b.n;
  const float d = b.mean - a.mean, f = b.n * __builtin_amdgcn_rcpf(n);  // 1-ulp reciprocal
  a.mean += d * f;
  a.m2 += b.m2 + d * d * a.n * f;
  a.n = n;
}

// Merge across the 64 lanes of a wave; lane 0 ends with the lanes merged in
// one fixed order (the lower lane's side first at every step).
__device__ __forceinline__ Moments wave_merge(Moments t) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    Moments o;
    o.n = __shfl_xor(t.n, off);
    o.mean = __shfl_xor(t.mean, off);
    o.m2 = __shfl_xor(t.m2, off);
    if (lane & off) {
      Moments s = o;
      merge(s, t);
      t = s;
    } else {
      merge(t, o);
    }
  }
  return t;
}

// Moments of the workgroup's threads (NT threads), the same on every thread.
template <int NT>
__device__ Moments block_merge(Moments t, Moments* lds) {
  t = wave_merge(t);
  __syncthreads();  // a previous call's readers are done with lds
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = t;
  __syncthreads();
  Moments r = lds[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) merge(r, lds[w]);
  return r;
}

template <class E, bool kVec>
struct GnIo {
  static constexpr int VW = kVec ? E::VW : 1;
  static constexpr size_t ES = 16 / E::VW;  // element size
  // vector v of the group starting at element `base`, raw
  using Raw = typename std::conditional<kVec, uint4, float>::type;
  static __device__ __forceinline__ Raw load(const void* x, size_t base, long long v) {
    if constexpr (kVec)
      return *(const uint4*)((const char*)x + (base + (size_t)v * VW) * ES);
    else
      return E::get(x, base + (size_t)v);
  }
  static __device__ __forceinline__ void unpack(const Raw& r, float* f) {
    if constexpr (kVec)
      E::unpack(r, f);
    else
      f[0] = r;
  }
  // The same, marking the raw words as rewritten first (an empty asm
  // statement, no instruction): otherwise the compiler reuses the floats of
  // an earlier unpack of the same words and keeps them live in the meantime,
  // which doubles the registers a thread needs for its values.
  static __device__ __forceinline__ void unpack_again(Raw& r, float* f) {
    if constexpr (kVec)
      asm volatile("" : "+v"(r.x), "+v"(r.y), "+v"(r.z), "+v"(r.w));
    else
      asm volatile("" : "+v"(r));
    unpack(r, f);
  }
  static __device__ __forceinline__ void store(void* y, size_t base, long long v, const float* f) {
    if constexpr (kVec)
      *(uint4*)((char*)y + (base + (size_t)v * VW) * ES) = E::pack(f);
    else
      E::put(y, base + (size_t)v, f[0]);
  }
};

// y = x a_c + b_c for vector v of the group, a_c = rstd gamma_c,
// b_c = beta_c - mean a_c (every element of a vector is in channel c).
template <class E, bool kVec>
__device__ __forceinline__ void gn_write(const GnArgs& a, int gin, size_t base, long long v, float* f, float mean,
                                         float rstd) {
  using IO = GnIo<E, kVec>;
  // the group's elements number below 2^31 (checked at launch): 32-bit division
  const int c = gin * a.Cg + (int)((unsigned)(v * IO::VW) / (unsigned)a.HW);
  const float ga = a.gamma ? E::get(a.gamma, c) : 1.f;
  const float be = a.beta ? E::get(a.beta, c) : 0.f;
  const float sc = rstd * ga, sh = be - mean * sc;
#pragma unroll
  for (int i = 0; i < IO::VW; ++i) f[i] = __builtin_fmaf(f[i], sc, sh);
  IO::store(a.y, base, v, f);
}

template <class E, bool kVec, int RV>
__global__ __launch_bounds__(kGnFusedThreads) void gn_fused_kernel(const GnArgs a) {
  using IO = GnIo<E, kVec>;
  constexpr int VW = IO::VW;
  __shared__ Moments lds[kGnFusedThreads / 64];
  const int tid = threadIdx.x;
  const int grp = blockIdx.x;
  const size_t base = (size_t)grp * a.L;
  const long long lv = a.L / VW;
  typename IO::Raw raw[RV];
#pragma unroll
  for (int k = 0; k < RV; ++k) {
    const long long v = tid + (long long)k * kGnFusedThreads;
    if (v < lv) raw[k] = IO::load(a.x, base, v);
  }
  // this thread's moments: mean first, then squared deviations
  float n = 0.f, s = 0.f;
#pragma unroll
  for (int k = 0; k < RV; ++k) {
    if (tid + (long long)k * kGnFusedThreads < lv) {
      float f[VW];
      IO::unpack(raw[k], f);
#pragma unroll
      for (int i = 0; i < VW; ++i) s += f[i];
      n += (float)VW;
    }
  }
  Moments t = {n, n > 0.f ? s / n : 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < RV; ++k) {
    if (tid + (long long)k * kGnFusedThreads < lv) {
      float f[VW];
      IO::unpack_again(raw[k], f);
#pragma unroll
      for (int i = 0; i < VW; ++i) t.m2 += (f[i] - t.mean) * (f[i] - t.mean);
    }
  }
  const Moments g = block_merge<kGnFusedThreads>(t, lds);
  const float rstd = 1.f / __builtin_sqrtf(g.m2 / (float)a.L + a.eps);
  const int gin = grp % a.G;
#pragma unroll
  for (int k = 0; k < RV; ++k) {
    const long long v = tid + (long long)k * kGnFusedThreads;
    if (v < lv) {
      float f[VW];
      IO::unpack_again(raw[k], f);
      gn_write<E, kVec>(a, gin, base, v, f, g.mean, rstd);
    }
  }
}

// Two-launch path, first launch: the moments of every slice.
template <class E, bool kVec>
__global__ __launch_bounds__(kGnSliceThreads) void gn_partial_kernel(const GnArgs a) {
  using IO = GnIo<E, kVec>;
  constexpr int VW = IO::VW;
  __shared__ Moments lds[kGnSliceThreads / 64];
  const int grp = blockIdx.x / a.S, sl = blockIdx.x - grp * a.S;
  const size_t base = (size_t)grp * a.L;
  const long long lv = a.L / VW;
  const long long v0 = (long long)sl * a.slice_vec;
  const long long v1 = v0 + a.slice_vec < lv ? v0 + a.slice_vec : lv;
  Moments t = {0.f, 0.f, 0.f};
  for (long long vb = v0 + threadIdx.x; vb < v1; vb += (long long)kGnSliceThreads * kGnSliceBatch) {
    typename IO::Raw raw[kGnSliceBatch];
#pragma unroll
    for (int k = 0; k < kGnSliceBatch; ++k) {
      const long long v = vb + (long long)k * kGnSliceThreads;
      if (v < v1) raw[k] = IO::load(a.x, base, v);
    }
    // the batch's moments by two passes over its values, then one merge
    float n = 0.f, s = 0.f;
#pragma unroll
    for (int k = 0; k < kGnSliceBatch; ++k) {
      if (vb + (long long)k * kGnSliceThreads < v1) {
        float f[VW];
        IO::unpack(raw[k], f);
#pragma unroll
        for (int i = 0; i < VW; ++i) s += f[i];
        n += (float)VW;
      }
    }
    Moments b = {n, s * __builtin_amdgcn_rcpf(n), 0.f};
#pragma unroll
    for (int k = 0; k < kGnSliceBatch; ++k) {
      if (vb + (long long)k * kGnSliceThreads < v1) {
        float f[VW];
        IO::unpack(raw[k], f);
#pragma unroll
        for (int i = 0; i < VW; ++i) b.m2 += (f[i] - b.mean) * (f[i] - b.mean);
      }
    }
    merge(t, b);
  }
  const Moments m = block_merge<kGnSliceThreads>(t, lds);
  if (threadIdx.x == 0) {
    a.ws[2 * (size_t)blockIdx.x] = tag(m.mean, a.epoch);
    a.ws[2 * (size_t)blockIdx.x + 1] = tag(m.m2, a.epoch);
  }
}

// Two-launch path, second launch: merge the group's slice moments, normalise
// this slice.
template <class E, bool kVec>
__global__ __launch_bounds__(kGnSliceThreads) void gn_apply_kernel(const GnArgs a) {
  using IO = GnIo<E, kVec>;
  constexpr int VW = IO::VW;
  __shared__ float2 coef;
  const int tid = threadIdx.x;
  const int grp = blockIdx.x / a.S, sl = blockIdx.x - grp * a.S;
  const size_t base = (size_t)grp * a.L;
  const long long lv = a.L / VW;
  if (tid < 64) {
    // lane j merges slices j, j + 64, ... in order, then the lanes merge
    Moments g = {0.f, 0.f, 0.f};
    for (int s = tid; s < a.S; s += 64) {
      const unsigned long long* w = a.ws + 2 * ((size_t)grp * a.S + s);
      const float2 p = make_float2(untag(w[0]), untag(w[1]));
      const long long s0 = (long long)s * a.slice_vec;
      const long long s1 = s0 + a.slice_vec < lv ? s0 + a.slice_vec : lv;
      const Moments m = {(float)((s1 - s0) * VW), p.x, p.y};
      merge(g, m);
    }
    g = wave_merge(g);
    if (tid == 0) coef = make_float2(g.mean, 1.f / __builtin_sqrtf(g.m2 / (float)a.L + a.eps));
  }
  __syncthreads();
  const float mean = coef.x, rstd = coef.y;
  const int gin = grp % a.G;
  const long long v0 = (long long)sl * a.slice_vec;
  const long long v1 = v0 + a.slice_vec < lv ? v0 + a.slice_vec : lv;
  for (long long vb = v0 + tid; vb < v1; vb += (long long)kGnSliceThreads * kGnSliceBatch) {
    typename IO::Raw raw[kGnSliceBatch];
#pragma unroll
    for (int k = 0; k < kGnSliceBatch; ++k) {
      const long long v = vb + (long long)k * kGnSliceThreads;
      if (v < v1) raw[k] = IO::load(a.x, base, v);
    }
#pragma unroll
    for (int k = 0; k < kGnSliceBatch; ++k) {
      const long long v = vb + (long long)k * kGnSliceThreads;
      if (v < v1) {
        float f[VW];
        IO::unpack(raw[k], f);
        gn_write<E, kVec>(a, gin, base, v, f, mean, rstd);
      }
    }
  }
}

// One-launch split form (the groups fill less of the chip than their data
// would need): S workgroups per group, each holding its slice in registers.
// A workgroup publishes its slice's moments as two tagged 64-bit words
// (value and call epoch in one word, written and read as relaxed agent-scope
// atomics: a reader sees either the old word or the whole new one, so no
// cache write-back or invalidation is needed) and waits until all S slots of
// its group carry this call's epoch.  The wait is bounded: a workgroup whose
// partners have not all published within spin_limit polls (they may not be
// resident yet) computes every slice's moments itself from x, with the same
// per-slice arithmetic, so the result is the same either way and no
// workgroup ever waits without end.
constexpr int kGnCoopThreads = 256, kGnCoopMaxRv = 8, kGnCoopMaxSlices = 64;

// Moments of slice s (vectors v0 + tid + k * NT), two passes per thread, merged
// over the workgroup; with `load` the slice is read into raw first.
template <class E, bool kVec, int RV, int NT>
__device__ Moments slice_moments(const GnArgs& a, size_t base, long long lv, int s,
                                 typename GnIo<E, kVec>::Raw (&raw)[RV], bool load, Moments* lds) {
  using IO = GnIo<E, kVec>;
  constexpr int VW = IO::VW;
  const int tid = threadIdx.x;
  const long long v0 = (long long)s * a.slice_vec;
  const long long v1 = v0 + a.slice_vec < lv ? v0 + a.slice_vec : lv;
  if (load) {
#pragma unroll
    for (int k = 0; k < RV; ++k) {
      const long long v = v0 + tid + (long long)k * NT;
      if (v < v1) raw[k] = IO::load(a.x, base, v);
    }
  }
  float n = 0.f, sum = 0.f;
#pragma unroll
  for (int k = 0; k < RV; ++k) {
    if (v0 + tid + (long long)k * NT < v1) {
      float f[VW];
      IO::unpack(raw[k], f);
#pragma unroll
      for (int i = 0; i < VW; ++i) sum += f[i];
      n += (float)VW;
    }
  }
  Moments t = {n, n > 0.f ? sum / n : 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < RV; ++k) {
    if (v0 + tid + (long long)k * NT < v1) {
      float f[VW];
      IO::unpack_again(raw[k], f);
#pragma unroll
      for (int i = 0; i < VW; ++i) t.m2 += (f[i] - t.mean) * (f[i] - t.mean);
    }
  }
  return block_merge<NT>(t, lds);
}

// (mean, rstd) of a group from its S slice moments, merged on wave 0 in a
// fixed order: lane j takes slices j, j + 64, ..., then the lanes merge.
template <int VW>
__device__ void merge_slices(const GnArgs& a, const float2* parts, long long lv, float2* coef) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    Moments g = {0.f, 0.f, 0.f};
    for (int s = tid; s < a.S; s += 64) {
      const float2 p = parts[s];
      const long long s0 = (long long)s * a.slice_vec;
      const long long s1 = s0 + a.slice_vec < lv ? s0 + a.slice_vec : lv;
      const Moments m = {(float)((s1 - s0) * VW), p.x, p.y};
      merge(g, m);
    }
    g = wave_merge(g);
    if (tid == 0) *coef = make_float2(g.mean, 1.f / __builtin_sqrtf(g.m2 / (float)a.L + a.eps));
  }
}

template <class E, bool kVec, int RV>
__global__ __launch_bounds__(kGnCoopThreads) void gn_coop_kernel(const GnArgs a) {
  using IO = GnIo<E, kVec>;
  constexpr int VW = IO::VW;
  __shared__ Moments lds[kGnCoopThreads / 64];
  __shared__ float2 parts[kGnCoopMaxSlices];
  __shared__ float2 coef;
  __shared__ int synced;
  const int tid = threadIdx.x;
  const int grp = blockIdx.x / a.S, sl = blockIdx.x - grp * a.S;
  const size_t base = (size_t)grp * a.L;
  const long long lv = a.L / VW;
  typename IO::Raw raw[RV];
  const Moments mine = slice_moments<E, kVec, RV, kGnCoopThreads>(a, base, lv, sl, raw, true, lds);
  if (tid == 0) {
    unsigned long long* w = a.ws + 2 * (size_t)blockIdx.x;
    __hip_atomic_store(w, tag(mine.mean, a.epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(w + 1, tag(mine.m2, a.epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < 64) {
    // lane j polls slot j of the group (S <= 64)
    unsigned long long* w = a.ws + 2 * ((size_t)grp * a.S + tid);
    unsigned long long w0 = 0, w1 = 0;
    bool ready = tid >= a.S;
    for (int i = 0; i <= a.spin_limit; ++i) {
      if (!ready) {
        w0 = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w1 = __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ready = (unsigned)(w0 >> 32) == a.epoch && (unsigned)(w1 >> 32) == a.epoch;
      }
      if (__all(ready) || i == a.spin_limit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (tid < a.S) parts[tid] = make_float2(untag(w0), untag(w1));
    const bool all_ready = __all(ready);
    if (tid == 0) synced = all_ready;
  }
  __syncthreads();
  if (synced) {
    merge_slices<VW>(a, parts, lv, &coef);
  } else {
    // partners not (yet) resident: every slice's moments from x, as they
    // would have computed them, then this slice again for the output
    for (int s = 0; s < a.S; ++s) {
      const Moments m = slice_moments<E, kVec, RV, kGnCoopThreads>(a, base, lv, s, raw, true, lds);
      if (tid == 0) parts[s] = make_float2(m.mean, m.m2);
    }
    __syncthreads();
    merge_slices<VW>(a, parts, lv, &coef);
    (void)slice_moments<E, kVec, RV, kGnCoopThreads>(a, base, lv, sl, raw, true, lds);
  }
  __syncthreads();
  const float mean = coef.x, rstd = coef.y;
  const int gin = grp % a.G;
  const long long v0 = (long long)sl * a.slice_vec;
  const long long v1 = v0 + a.slice_vec < lv ? v0 + a.slice_vec : lv;
#pragma unroll
  for (int k = 0; k < RV; ++k) {
    const long long v = v0 + tid + (long long)k * kGnCoopThreads;
    if (v < v1) {
      float f[VW];
      IO::unpack_again(raw[k], f);
      gn_write<E, kVec>(a, gin, base, v, f, mean, rstd);
    }
  }
}

// The launch plan of one problem: fused (RV vectors per thread) or two
// launches over S slices per group.
struct GnPlan {
  bool vec;
  int rv;            // > 0: fused with rv vectors per thread
  int coop_rv;       // > 0: one-launch split form with coop_rv vectors per thread
  long long s;       // slices per group (split forms)
  long long slice_vec;
  size_t ws_bytes;   // workspace the plan needs
};

// ATTN_GN_PATH=split / fused / coop forces a form (for measurements; fused
// and coop only where they fit).
int forced_path() {
  const char* e = std::getenv("ATTN_GN_PATH");
  if (!e) return 0;
  if (!std::strcmp(e, "split")) return 1;
  if (!std::strcmp(e, "fused")) return 2;
  if (!std::strcmp(e, "coop")) return 3;
  return 0;
}

// Epoch of a call: nonzero and new for every call (a zero-filled workspace
// holds epoch 0 and earlier calls' words hold earlier epochs; the counter
// repeats only after 2^32 - 1 calls).
unsigned next_epoch() {
  static std::atomic<unsigned> counter{0};
  unsigned e = counter.fetch_add(1u, std::memory_order_relaxed) + 1u;
  if (e == 0u) e = counter.fetch_add(1u, std::memory_order_relaxed) + 1u;
  return e;
}

// Polls before a one-launch split workgroup computes its group's moments on
// its own (ATTN_GN_SPIN overrides, e.g. 0 to exercise that path).
int spin_limit() {
  const char* e = std::getenv("ATTN_GN_SPIN");
  return e ? std::atoi(e) : (1 << 16);
}

// Workgroups of `kern` (256 threads) resident at once on the current device.
int resident_wgs(const void* kern) {
  int dev = 0, per_cu = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kGnCoopThreads, 0) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return per_cu * cus;
}

template <class E, bool kVec>
const void* coop_kernel(int rv) {
  switch (rv) {
    case 1: return (const void*)gn_coop_kernel<E, kVec, 1>;
    case 2: return (const void*)gn_coop_kernel<E, kVec, 2>;
    case 4: return (const void*)gn_coop_kernel<E, kVec, 4>;
    default: return (const void*)gn_coop_kernel<E, kVec, 8>;
  }
}

// The one-launch split form tells this call's slice moments from earlier
// ones by an epoch taken on the host at launch; a captured graph would replay
// the same epoch over words its previous replay left, so a call on a stream
// being captured takes the stream-ordered two-launch form instead.
template <class E>
GnPlan gn_plan(const GroupNormProblem& p, bool capturing) {
  GnPlan pl;
  pl.vec = p.HW % E::VW == 0 && ((uintptr_t)p.x & 15u) == 0 && ((uintptr_t)p.y & 15u) == 0;
  const int VW = pl.vec ? E::VW : 1;
  const long long L = (long long)(p.C / p.G) * p.HW, lv = L / VW;
  const long long ng = (long long)p.N * p.G;
  pl.rv = 0;
  pl.coop_rv = 0;
  pl.s = 1;
  pl.slice_vec = lv;
  pl.ws_bytes = 0;
  // One launch when the group fits the registers and either the groups fill
  // the chip (a workgroup of 1024 threads per group, one per CU or more) or
  // they are small (two vectors per thread at most): a single workgroup
  // moves only ~10-20 GB/s against HBM latency, so a few large groups go
  // faster over many workgroups in two launches.
  const int forced = forced_path();
  int rv_fit = 0;
  for (int rv = 1; rv <= kGnMaxRv && !rv_fit; rv *= 2)
    if ((long long)rv * kGnFusedThreads >= lv) rv_fit = rv;
  if (rv_fit && forced != 1 && forced != 3 && (forced == 2 || ng >= kGnFusedMinGroups || rv_fit <= 2)) {
    pl.rv = rv_fit;
    return pl;
  }
  // Split forms: the workspace holds 16 bytes of tagged moments per slice.
  pl.coop_rv = 0;
  // not in place either: a workgroup whose wait runs out recomputes its
  // partners' moments from x, which an in-place partner may have overwritten
  if (forced != 1 && !capturing && p.x != p.y) {
    // one launch: about kGnSliceTarget workgroups, slices of at most
    // kGnCoopMaxRv vectors per thread, at most kGnCoopMaxSlices per group,
    // all workgroups resident at once
    const long long cap_slice = (long long)kGnCoopThreads * kGnCoopMaxRv;
    long long sc = (kGnSliceTarget + ng - 1) / ng;
    const long long s_min = (lv + cap_slice - 1) / cap_slice;
    const long long s_max = (lv + kGnCoopThreads - 1) / kGnCoopThreads;  // a vector per thread at least
    if (sc > s_max) sc = s_max;
    if (sc < s_min) sc = s_min;
    if (sc < 1) sc = 1;
    const long long sv = (lv + sc - 1) / sc;
    sc = (lv + sv - 1) / sv;
    int rv = 1;
    while ((long long)rv * kGnCoopThreads < sv) rv *= 2;
    if (sc >= 2 && sc <= kGnCoopMaxSlices && rv <= kGnCoopMaxRv &&
        ng * sc <= resident_wgs(pl.vec ? coop_kernel<E, true>(rv) : coop_kernel<E, false>(rv))) {
      pl.coop_rv = rv;
      pl.s = sc;
      pl.slice_vec = sv;
      pl.ws_bytes = (size_t)(ng * sc) * 16;
      return pl;
    }
  }
  // two launches: about kGnSliceTarget workgroups, each slice at least one
  // full batch of vectors per thread
  const long long min_slice = (long long)kGnSliceThreads * kGnSliceBatch;
  long long s = (kGnSliceTarget + ng - 1) / ng;
  const long long most = (lv + min_slice - 1) / min_slice;
  if (s > most) s = most;
  if (s < 1) s = 1;
  pl.slice_vec = (lv + s - 1) / s;
  pl.s = (lv + pl.slice_vec - 1) / pl.slice_vec;  // every slice non-empty
  pl.ws_bytes = (size_t)(ng * pl.s) * 16;
  return pl;
}

template <class E, bool kVec, int RV>
void launch_fused(const GnArgs& a, long long ng, hipStream_t st) {
  hipLaunchKernelGGL((gn_fused_kernel<E, kVec, RV>), dim3((unsigned)ng), dim3(kGnFusedThreads), 0, st, a);
}

template <class E, bool kVec>
hipError_t launch_gn_t(const GroupNormProblem& p, const GnPlan& pl) {
  GnArgs a;
  a.x = p.x;
  a.gamma = p.gamma;
  a.beta = p.beta;
  a.y = p.y;
  a.ws = (unsigned long long*)p.workspace;
  a.epoch = next_epoch();
  a.spin_limit = spin_limit();
  a.HW = p.HW;
  a.G = p.G;
  a.Cg = p.C / p.G;
  a.L = (long long)a.Cg * p.HW;
  a.S = (int)pl.s;
  a.slice_vec = pl.slice_vec;
  a.eps = p.eps;
  const long long ng = (long long)p.N * p.G;
  if (a.L >= 0x7fffffffLL) return hipErrorInvalidValue;
  if (pl.rv > 0) {
    if (ng > 0x7fffffffLL) return hipErrorInvalidValue;
    switch (pl.rv) {
      case 1: launch_fused<E, kVec, 1>(a, ng, p.stream); break;
      case 2: launch_fused<E, kVec, 2>(a, ng, p.stream); break;
      case 4: launch_fused<E, kVec, 4>(a, ng, p.stream); break;
      case 8: launch_fused<E, kVec, 8>(a, ng, p.stream); break;
      default: launch_fused<E, kVec, 16>(a, ng, p.stream); break;
    }
    return hipGetLastError();
  }
  const long long grid = ng * pl.s;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (pl.coop_rv > 0) {
    switch (pl.coop_rv) {
      case 1: hipLaunchKernelGGL((gn_coop_kernel<E, kVec, 1>), dim3((unsigned)grid), dim3(kGnCoopThreads), 0, p.stream, a); break;
      case 2: hipLaunchKernelGGL((gn_coop_kernel<E, kVec, 2>), dim3((unsigned)grid), dim3(kGnCoopThreads), 0, p.stream, a); break;
      case 4: hipLaunchKernelGGL((gn_coop_kernel<E, kVec, 4>), dim3((unsigned)grid), dim3(kGnCoopThreads), 0, p.stream, a); break;
      default: hipLaunchKernelGGL((gn_coop_kernel<E, kVec, 8>), dim3((unsigned)grid), dim3(kGnCoopThreads), 0, p.stream, a); break;
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gn_partial_kernel<E, kVec>), dim3((unsigned)grid), dim3(kGnSliceThreads), 0, p.stream, a);
  hipLaunchKernelGGL((gn_apply_kernel<E, kVec>), dim3((unsigned)grid), dim3(kGnSliceThreads), 0, p.stream, a);
  return hipGetLastError();
}

// Whether work on `st` is being captured into a graph (an error counts as
// yes: the two-launch form is correct either way).
bool stream_capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return true;
  return cs != hipStreamCaptureStatusNone;
}

template <class E>
hipError_t launch_gn_e(const GroupNormProblem& p) {
  const GnPlan pl = gn_plan<E>(p, stream_capturing(p.stream));
  if (pl.ws_bytes > p.workspace_bytes || (pl.ws_bytes && !p.workspace)) return hipErrorInvalidValue;
  return pl.vec ? launch_gn_t<E, true>(p, pl) : launch_gn_t<E, false>(p, pl);
}

// Enough for the plan of either kind of call, captured or not.
template <class E>
size_t gn_ws_e(const GroupNormProblem& p) {
  const size_t a = gn_plan<E>(p, false).ws_bytes, b = gn_plan<E>(p, true).ws_bytes;
  return a > b ? a : b;
}

// ---------------------------------------------------------------------------
// GELU-gated product: h [rows][2F] -> out [rows][F], out = h[:, :F] *
// gelu(h[:, F:]).  Each thread takes kGeVecs output vectors of 16 bytes: two
// 16-byte loads (value and gate) and one store per vector, float arithmetic.
// One vector per thread in 256-thread workgroups measured fastest (2, 4 and 8
// per thread, and 128 to 1024 threads, were 0-30 % slower).
// ---------------------------------------------------------------------------
constexpr int kGeThreads = 256, kGeVecs = 1;

// gelu(g) = g Phi(g) with Phi(g) = erfc(-g / sqrt 2) / 2, erfc taken for the
// non-negative argument z = |g| / sqrt 2 (Phi(g) = 1 - erfc(z) / 2 for g >= 0)
// from the Chebyshev fit erfc(z) ~ t exp(-z^2 + P(t)), t = 1 / (1 + z / 2),
// P of degree 9, of Press et al., Numerical Recipes in C (2nd ed.), section
// 6.2, whose fractional error stays below 1.2e-7 for every z: relative
// accuracy in the lower tail too, at about 20 operations (the library erff
// costs about 55).  The exponent is evaluated in base 2 with log2(e) and the
// factor 1/2 folded into P's coefficients: erfc(z) / 2 = t 2^(P'(t) - g^2 log2(e) / 2).
constexpr double kL2E = 1.4426950408889634;
constexpr float kErfcP[10] = {
    (float)(-1.26551223 * kL2E - 1.0), (float)(1.00002368 * kL2E), (float)(0.37409196 * kL2E),
    (float)(0.09678418 * kL2E),        (float)(-0.18628806 * kL2E), (float)(0.27886807 * kL2E),
    (float)(-1.13520398 * kL2E),       (float)(1.48851587 * kL2E),  (float)(-0.82215223 * kL2E),
    (float)(0.17087277 * kL2E)};

__device__ __forceinline__ float gelu(float g) {
  const float z = __builtin_fabsf(g) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, z, 1.f));
  float p = kErfcP[9];
#pragma unroll
  for (int i = 8; i >= 0; --i) p = __builtin_fmaf(p, t, kErfcP[i]);
  const float half_erfc = t * __builtin_amdgcn_exp2f(__builtin_fmaf(g * (float)(-0.5 * kL2E), g, p));
  return g * (g < 0.f ? half_erfc : 1.f - half_erfc);
}

template <class E, bool kVec>
__global__ __launch_bounds__(kGeThreads) void geglu_kernel(const void* __restrict__ h, void* __restrict__ out,
                                                           int nvec, int fv, int F) {
  constexpr int VW = kVec ? E::VW : 1;
  constexpr size_t ES = 16 / E::VW;  // element size
  // output vector i = r fv + j / VW of row r; a thread's vectors are kGeThreads apart
  const int first = blockIdx.x * (kGeThreads * kGeVecs) + threadIdx.x;
  int r[kGeVecs], j[kGeVecs];
  r[0] = first / fv;
  j[0] = first - r[0] * fv;
#pragma unroll
  for (int u = 1; u < kGeVecs; ++u) {
    r[u] = r[u - 1];
    j[u] = j[u - 1] + kGeThreads;
    if (j[u] >= fv) {
      const int q = j[u] / fv;
      r[u] += q;
      j[u] -= q * fv;
    }
  }
  float val[kGeVecs][VW], gate[kGeVecs][VW];
#pragma unroll
  for (int u = 0; u < kGeVecs; ++u) {
    if (first + u * kGeThreads < nvec) {
      const size_t src = (size_t)r[u] * 2 * F + (size_t)j[u] * VW;
      if constexpr (kVec) {
        E::unpack(*(const uint4*)((const char*)h + src * ES), val[u]);
        E::unpack(*(const uint4*)((const char*)h + (src + F) * ES), gate[u]);
      } else {
        val[u][0] = E::get(h, src);
        gate[u][0] = E::get(h, src + F);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kGeVecs; ++u) {
    if (first + u * kGeThreads < nvec) {
      float o[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) o[e] = val[u][e] * gelu(gate[u][e]);
      const size_t dst = (size_t)r[u] * F + (size_t)j[u] * VW;
      if constexpr (kVec)
        *(uint4*)((char*)out + dst * ES) = E::pack(o);
      else
        E::put(out, dst, o[0]);
    }
  }
}

template <class E>
hipError_t launch_geglu_e(const GegluProblem& p) {
  const bool vec = p.F % E::VW == 0 && ((uintptr_t)p.h & 15u) == 0 && ((uintptr_t)p.out & 15u) == 0;
  const int VW = vec ? E::VW : 1;
  const int fv = p.F / VW;
  const long long nvec = (long long)p.rows * fv;
  if (nvec + (long long)kGeThreads * kGeVecs > 0x7fffffffLL) return hipErrorInvalidValue;
  const long long per_wg = (long long)kGeThreads * kGeVecs;
  const long long grid = (nvec + per_wg - 1) / per_wg;
  if (vec)
    hipLaunchKernelGGL((geglu_kernel<E, true>), dim3((unsigned)grid), dim3(kGeThreads), 0, p.stream, p.h, p.out,
                       (int)nvec, fv, p.F);
  else
    hipLaunchKernelGGL((geglu_kernel<E, false>), dim3((unsigned)grid), dim3(kGeThreads), 0, p.stream, p.h, p.out,
                       (int)nvec, fv, p.F);
  return hipGetLastError();
}

// Scratch of the allocation-free group normalisation (attn_group_norm_static):
// one array per device, the workspace of every such call on that device.
// Zero at load (static storage), which is the state the split forms expect
// before their first use; they leave it ready for the next call.  Host code
// must not pass the array's name to a kernel (on the host it only stands for
// the symbol): its device address comes from hipGetSymbolAddress below.
__device__ __align__(256) unsigned long long scratch[kGnStaticScratchBytes / 8];

}  // namespace

hipError_t group_norm_static_scratch(void** ptr) {
  // device address of `scratch`, looked up once per device with that device
  // current (every device holds its own copy at its own address)
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_group_norm(const GroupNormProblem& p) {
  switch (p.dt) {
    case ATTN_F16: return launch_gn_e<EF16>(p);
    case ATTN_BF16: return launch_gn_e<EBF16>(p);
    default: return launch_gn_e<EF32>(p);
  }
}

size_t group_norm_workspace(const GroupNormProblem& p) {
  switch (p.dt) {
    case ATTN_F16: return gn_ws_e<EF16>(p);
    case ATTN_BF16: return gn_ws_e<EBF16>(p);
    default: return gn_ws_e<EF32>(p);
  }
}

hipError_t launch_geglu(const GegluProblem& p) {
  switch (p.dt) {
    case ATTN_F16: return launch_geglu_e<EF16>(p);
    case ATTN_BF16: return launch_geglu_e<EBF16>(p);
    default: return launch_geglu_e<EF32>(p);
  }
}

}  // namespace attn
