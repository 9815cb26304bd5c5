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
#include <hip/hip_cooperative_groups.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "attn_internal.h"

namespace attn {
namespace {

namespace cg = cooperative_groups;

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
// span of L = (C/G) HW elements.  Every group is cut into S slices of
// consecutive 16-byte vectors, one workgroup per slice.  A workgroup reduces
// its slice to (count, mean, M2) -- per thread, then across the workgroup with
// the pairwise update (n, m, M2) + (n', m', M2') = (n + n', m + d n'/(n + n'),
// M2 + M2' + d^2 n n'/(n + n')), d = m' - m -- and, when S > 1, publishes the
// pair in a small workspace, waits at a grid barrier (cooperative launch: all
// workgroups are resident) and merges its group's S pairs in slice order, so
// every workgroup of a group derives the same mean and 1/sqrt(var + eps).  It
// then writes its slice.  With kResident the slice stays in registers between
// the two phases (x is read once); otherwise it is read a second time.
// ---------------------------------------------------------------------------
constexpr int kGnThreads = 256;
constexpr int kGnResidentVecs = 4;  // 16-byte vectors per thread kept in registers

struct GnArgs {
  const void* x;
  const void* gamma;  // [C] or null
  const void* beta;   // [C] or null
  void* y;
  float2* ws;          // [grid] (mean, M2) per slice, used when S > 1
  long long L;         // elements per group
  long long slice_vec; // vectors per slice (the last slice of a group may be shorter)
  int C, HW, G, Cg, S;
  float eps;
};

struct Moments {
  float n, mean, m2;
};

__device__ __forceinline__ void merge(Moments& a, const Moments& b) {
  const float n = a.n + b.n;
  if (b.n == 0.f) return;
  if (a.n == 0.f) {
    a = b;
    return;
  }
  const float d = b.mean - a.mean, f = b.n / n;
  a.mean += d * f;
  a.m2 += b.m2 + d * d * a.n * f;
  a.n = n;
}

// Moments of the workgroup's threads, merged in a fixed order; the result is
// returned to every thread.
__device__ Moments block_merge(Moments t, Moments* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    Moments o;
    o.n = __shfl_xor(t.n, off);
    o.mean = __shfl_xor(t.mean, off);
    o.m2 = __shfl_xor(t.m2, off);
    // the lower lane keeps its own side first: lane 0 ends with one fixed order
    if (lane & off) {
      Moments s = o;
      merge(s, t);
      t = s;
    } else {
      merge(t, o);
    }
  }
  if (lane == 0) lds[wave] = t;
  __syncthreads();
  Moments r = lds[0];
#pragma unroll
  for (int w = 1; w < kGnThreads / 64; ++w) merge(r, lds[w]);
  __syncthreads();  // lds may be reused
  return r;
}

template <class E, bool kVec>
struct GnIo {
  static constexpr int VW = kVec ? E::VW : 1;
  // vector v of a group starting at element `base`: VW floats
  static __device__ __forceinline__ void load(const void* x, size_t base, long long v, float* f) {
    if constexpr (kVec) {
      E::unpack(*(const uint4*)((const char*)x + (base + (size_t)v * VW) * sizeof_elem()), f);
    } else {
      f[0] = E::get(x, base + (size_t)v);
    }
  }
  static __device__ __forceinline__ void store(void* y, size_t base, long long v, const float* f) {
    if constexpr (kVec) {
      *(uint4*)((char*)y + (base + (size_t)v * VW) * sizeof_elem()) = E::pack(f);
    } else {
      E::put(y, base + (size_t)v, f[0]);
    }
  }
  static __device__ __forceinline__ constexpr size_t sizeof_elem() { return 16 / E::VW; }
};

template <class E, bool kSplit, bool kResident, bool kVec>
__global__ __launch_bounds__(kGnThreads) void group_norm_kernel(const GnArgs a) {
  using IO = GnIo<E, kVec>;
  constexpr int VW = IO::VW;
  __shared__ Moments lds[kGnThreads / 64];
  __shared__ float2 coef;  // (mean, rstd) of the group
  const int tid = threadIdx.x;
  const int grp = blockIdx.x / a.S, sl = blockIdx.x - grp * a.S;
  const size_t base = (size_t)grp * a.L;  // first element of the group
  const long long lv = a.L / VW;          // vectors per group
  const long long v0 = (long long)sl * a.slice_vec;
  const long long v1 = v0 + a.slice_vec < lv ? v0 + a.slice_vec : lv;

  // phase 1: moments of this thread's vectors (each vector reduced on its
  // own first, then merged), then of the workgroup
  float xr[kResident ? kGnResidentVecs : 1][VW];
  Moments t = {0.f, 0.f, 0.f};
  auto add_vector = [&](const float* f) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VW; ++i) s += f[i];
    Moments m;
    m.n = (float)VW;
    m.mean = s * (1.f / VW);
    m.m2 = 0.f;
#pragma unroll
    for (int i = 0; i < VW; ++i) m.m2 += (f[i] - m.mean) * (f[i] - m.mean);
    merge(t, m);
  };
  if constexpr (kResident) {
#pragma unroll
    for (int k = 0; k < kGnResidentVecs; ++k) {
      const long long v = v0 + tid + (long long)k * kGnThreads;
      if (v < v1) IO::load(a.x, base, v, xr[k]);
    }
#pragma unroll
    for (int k = 0; k < kGnResidentVecs; ++k)
      if (v0 + tid + (long long)k * kGnThreads < v1) add_vector(xr[k]);
  } else {
    for (long long v = v0 + tid; v < v1; v += kGnThreads) {
      float f[VW];
      IO::load(a.x, base, v, f);
      add_vector(f);
    }
  }
  const Moments wg = block_merge(t, lds);

  if (tid == 0 && !kSplit) coef = make_float2(wg.mean, 1.f / __builtin_sqrtf(wg.m2 / (float)a.L + a.eps));
  if constexpr (kSplit) {
    if (tid == 0) a.ws[blockIdx.x] = make_float2(wg.mean, wg.m2);
    cg::this_grid().sync();
    if (tid < 64) {
      // lane j merges slices j, j + 64, ... of the group in order, then the
      // lanes merge pairwise; lane 0 holds the group's moments
      Moments g = {0.f, 0.f, 0.f};
      for (int s = tid; s < a.S; s += 64) {
        const float2 p = a.ws[(size_t)grp * a.S + s];
        const long long s0 = (long long)s * a.slice_vec;
        const long long s1 = s0 + a.slice_vec < lv ? s0 + a.slice_vec : lv;
        Moments m = {(float)((s1 - s0) * VW), p.x, p.y};
        merge(g, m);
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        Moments o;
        o.n = __shfl_xor(g.n, off);
        o.mean = __shfl_xor(g.mean, off);
        o.m2 = __shfl_xor(g.m2, off);
        if (tid & off) {
          Moments s = o;
          merge(s, g);
          g = s;
        } else {
          merge(g, o);
        }
      }
      if (tid == 0) coef = make_float2(g.mean, 1.f / __builtin_sqrtf(g.m2 / (float)a.L + a.eps));
    }
  }
  __syncthreads();
  const float mean = coef.x, rstd = coef.y;

  // phase 2: y = x a_c + b_c with a_c = rstd gamma_c, b_c = beta_c - mean a_c
  const int gin = grp % a.G;  // group index within the sample
  auto write_vector = [&](long long v, float* f) {
    const int c = gin * a.Cg + (int)((v * VW) / a.HW);  // every element of a vector is in one channel
    const float ga = a.gamma ? E::get(a.gamma, c) : 1.f;
    const float be = a.beta ? E::get(a.beta, c) : 0.f;
    const float sc = rstd * ga, sh = be - mean * sc;
#pragma unroll
    for (int i = 0; i < VW; ++i) f[i] = f[i] * sc + sh;
    IO::store(a.y, base, v, f);
  };
  if constexpr (kResident) {
#pragma unroll
    for (int k = 0; k < kGnResidentVecs; ++k) {
      const long long v = v0 + tid + (long long)k * kGnThreads;
      if (v < v1) write_vector(v, xr[k]);
    }
  } else {
    for (long long v = v0 + tid; v < v1; v += kGnThreads) {
      float f[VW];
      IO::load(a.x, base, v, f);
      write_vector(v, f);
    }
  }
}

// Workgroups a cooperative launch of `kern` can keep resident on the current
// device (cached per device and kernel).
int resident_capacity(const void* kern) {
  static std::mutex mu;
  static const void* keys[64];
  static int devs[64], vals[64];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < used; ++i)
      if (keys[i] == kern && devs[i] == dev) return vals[i];
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kGnThreads, 0) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int cap = per_cu * cus;
  std::lock_guard<std::mutex> g(mu);
  if (used < 64) {
    keys[used] = kern;
    devs[used] = dev;
    vals[used] = cap;
    ++used;
  }
  return cap;
}

template <class E, bool kVec>
hipError_t launch_gn_t(const GroupNormProblem& p) {
  constexpr int VW = kVec ? E::VW : 1;
  GnArgs a;
  a.x = p.x;
  a.gamma = p.gamma;
  a.beta = p.beta;
  a.y = p.y;
  a.ws = (float2*)p.workspace;
  a.C = p.C;
  a.HW = p.HW;
  a.G = p.G;
  a.Cg = p.C / p.G;
  a.L = (long long)a.Cg * p.HW;
  a.eps = p.eps;
  const long long ng = (long long)p.N * p.G;  // groups
  const long long lv = a.L / VW;               // vectors per group
  const long long res_vecs = (long long)kGnThreads * kGnResidentVecs;
  const long long s_res = (lv + res_vecs - 1) / res_vecs;  // slices for register residency

  const void* k_split_res = (const void*)group_norm_kernel<E, true, true, kVec>;
  const void* k_split_str = (const void*)group_norm_kernel<E, true, false, kVec>;
  const long long max_grid = (long long)kGroupNormWorkspaceBytes / sizeof(float2);
  // Slices per group.  Groups that fit one workgroup's registers get one
  // workgroup (no barrier).  Larger groups are split -- when a workspace is
  // given and the chip has room -- into at least s_res slices (x is then read
  // once), as many as fill the resident workgroups, at most one vector per
  // thread; groups too large for the resident grid are streamed (read twice).
  long long s = 1;
  bool resident = s_res == 1;
  if (s_res > 1 && p.workspace && ng > 0) {
    const int cap = resident_capacity(k_split_res);
    const long long most = (lv + kGnThreads - 1) / kGnThreads;
    if (s_res * ng <= cap && s_res * ng <= max_grid) {
      const long long fill = cap / ng;
      s = fill < most ? fill : most;
      if (s < s_res) s = s_res;
      resident = true;
    } else {
      const int cap_str = resident_capacity(k_split_str);
      s = cap_str / ng;
      if (s * ng > max_grid) s = max_grid / ng;
      if (s < 1) s = 1;
      resident = false;
    }
  }
  a.slice_vec = (lv + s - 1) / s;
  s = (lv + a.slice_vec - 1) / a.slice_vec;  // every slice non-empty
  a.S = (int)s;
  const long long grid = ng * s;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;

  if (s == 1) {
    if (resident)
      hipLaunchKernelGGL((group_norm_kernel<E, false, true, kVec>), dim3((unsigned)grid), dim3(kGnThreads), 0,
                         p.stream, a);
    else
      hipLaunchKernelGGL((group_norm_kernel<E, false, false, kVec>), dim3((unsigned)grid), dim3(kGnThreads), 0,
                         p.stream, a);
    return hipGetLastError();
  }
  if (grid > max_grid) return hipErrorInvalidValue;
  void* args[] = {&a};
  return hipLaunchCooperativeKernel(resident ? k_split_res : k_split_str, dim3((unsigned)grid), dim3(kGnThreads),
                                    args, 0, p.stream);
}

template <class E>
hipError_t launch_gn_e(const GroupNormProblem& p) {
  const bool vec = p.HW % E::VW == 0 && ((uintptr_t)p.x & 15u) == 0 && ((uintptr_t)p.y & 15u) == 0;
  return vec ? launch_gn_t<E, true>(p) : launch_gn_t<E, false>(p);
}

// ---------------------------------------------------------------------------
// GELU-gated product: h [rows][2F] -> out [rows][F], out = h[:, :F] *
// gelu(h[:, F:]).  Each thread takes kGeVecs output vectors of 16 bytes: two
// 16-byte loads (value and gate) and one store per vector, float arithmetic.
// ---------------------------------------------------------------------------
constexpr int kGeThreads = 256, kGeVecs = 2;

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

}  // namespace

hipError_t launch_group_norm(const GroupNormProblem& p) {
  switch (p.dt) {
    case ATTN_F16: return launch_gn_e<EF16>(p);
    case ATTN_BF16: return launch_gn_e<EBF16>(p);
    default: return launch_gn_e<EF32>(p);
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
