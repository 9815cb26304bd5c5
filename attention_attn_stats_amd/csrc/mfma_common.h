// Matrix-core building blocks shared by the attention kernels for gfx950
// (CDNA4): vector types, the two 16-bit element types with their MFMA shapes
// and rounding, buffer-resource loads, the transposing LDS read, the
// XCD-aware workgroup order and cross-lane exchanges.
#ifndef ATTN_MFMA_COMMON_H
#define ATTN_MFMA_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
namespace {

typedef short s4v __attribute__((ext_vector_type(4)));
typedef short s8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef __bf16 b2v __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Element-type traits: the two MFMA shapes used, rounding of fp32 to the
// 16-bit type (round to nearest even) and back.
struct F16 {
  static __device__ __forceinline__ f4v mma16(s8v a, s8v b, f4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f16v mma32(s8v a, s8v b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, h2v));
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(h2v, w)[0];
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(h2v, w)[1];
  }
  static constexpr uint16_t kOne = 0x3C00;
  static constexpr uint16_t kMinus2p15 = 0xF800;  // -32768
  // A row sum of fp16-rounded P is within 2^-11 (relative) of the exact sum,
  // inside the 1e-3 bound on l, so the single pass may report the sum its
  // V ones column gives.
  static constexpr bool kRoundedSumOk = true;
  // packed 16-bit max instructions exist for this type
  static constexpr bool kPackedMax = true;
};

struct BF16 {
  static __device__ __forceinline__ f4v mma16(s8v a, s8v b, f4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8v, a), __builtin_bit_cast(b8v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f16v mma32(s8v a, s8v b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8v, a), __builtin_bit_cast(b8v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, b2v));
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
  static constexpr uint16_t kOne = 0x3F80;
  static constexpr uint16_t kMinus2p15 = 0xC700;  // -32768
  // bf16 rounding (2^-8) is too coarse for a reported l: sum in fp32 as well.
  static constexpr bool kRoundedSumOk = false;
  static constexpr bool kPackedMax = false;
};

constexpr int kModeFlash = 0;    // online softmax, O only
constexpr int kModeFlashML = 1;  // online softmax, O and (m, l)
constexpr int kModePV = 2;       // softmax from given (m, l), O only
constexpr int kModeStats = 3;    // (m, l) only: the first pass of the partially fused form
constexpr int kModePVScores = 4; // as kModePV, the logits read from a stored A instead of Q K^T

// max of two pairs of non-negative fp16 values (v_pk_maximum3_f16 from chains)
__device__ __forceinline__ uint32_t pmax(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(__builtin_bit_cast(h2v, a), __builtin_bit_cast(h2v, b)));
}
__device__ __forceinline__ float pmax_halves(uint32_t a) {
  const h2v v = __builtin_bit_cast(h2v, a);
  return (float)__builtin_elementwise_maximum(v[0], v[1]);
}

// An MFMA result, copied after 16 wait states: for its first read after code
// that branches.  The compiler counts the wait states such a read needs after
// the MFMA along one of the paths into the reading block only; 16 of its own,
// then a copy, cover every path (a 32x32x16 result read too early on the
// other path is stale).
__device__ __forceinline__ float mfma_settled(float x) {
  float y;
  asm volatile("s_nop 7\n\ts_nop 7\n\tv_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their no-wait maxima)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Raw buffer resource over `bytes` bytes at p (stride 0): loads at offsets
// at or past `bytes` return zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, int voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
}

typedef uint16_t __attribute__((address_space(3))) lds_u16;

__device__ __forceinline__ s4v lds_read_tr16(const uint16_t* p) {
  // generic -> LDS address space; the pointer is known to point into __shared__
  const lds_u16* lp = (const lds_u16*)(uintptr_t)(uint32_t)(uintptr_t)p;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s4v __attribute__((address_space(3)))*)lp);
}

// Workgroup index -> logical tile, keeping consecutive tiles (same head, so
// the same K and V) on one XCD: the hardware deals workgroups to the 8 XCDs
// round robin.
__device__ __forceinline__ int xcd_tile(int nwg) {
  int w = blockIdx.x;
  if ((nwg & 7) == 0) w = (w & 7) * (nwg >> 3) + (w >> 3);
  return w;
}

// Cross-lane exchanges.  v_permlane16_swap exchanges the odd 16-lane rows of
// its first operand with the even rows of its second; v_permlane32_swap the
// upper half of the first with the lower half of the second.  Swapping a
// value with itself is written as inline asm: this compiler's optimizer
// treats the two results of the swap builtins as interchangeable in that case
// and folds a reduction over them away.  The leading s_nop covers the wait
// states a swap needs after a vector-ALU write of its inputs.
// over lanes l and l ^ 32
template <class Op>
__device__ __forceinline__ float pair_reduce(float x, Op op) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float pair_max32(float x) {
  return pair_reduce(x, [](float a, float b) { return __builtin_fmaxf(a, b); });
}
__device__ __forceinline__ float pair_sum32(float x) {
  return pair_reduce(x, [](float a, float b) { return a + b; });
}
// 16-lane-row exchange of two distinct values: a <- (A.row0, B.row0, A.row2,
// B.row2), b <- (A.row1, B.row1, A.row3, B.row3).
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

}  // namespace
}  // namespace attn

#endif
