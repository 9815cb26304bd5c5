// Matrix-core attention kernels for gfx950 (CDNA4): fp16 / bf16 operands,
// fp32 accumulation and fp32 softmax state.
//
// Method: "Speed Is All You Need: On-Device Acceleration of Large Diffusion
// Models via GPU-Aware Optimizations" (Chen et al.), news write-up, section on
// improving attention efficiency.  Two forms of O = softmax(scale Q K^T) V:
//   * partially fused softmax: stats_kernel reduces every row of
//     A = scale Q K^T to (m, l) -- the N x 2 tensor -- with the row's keys cut
//     into blocks that are reduced separately and merged in the same launch;
//     fwd_kernel<.., kModePV> then applies the softmax inside the product with
//     V.  A is recomputed from Q and K on chip, never stored.
//   * FlashAttention: fwd_kernel<.., kModeFlash*> walks the key blocks once
//     with a running max and running sum (exact online softmax).
//
// Shared design (all kernels):
//   * Scores are formed transposed, S^T = K Q^T, with the 16x16x32 MFMA; a
//     head-dim remainder of 8 or 16 takes one more 16x16x32 step whose
//     missing dims are zero in the Q operand.  In the
//     MFMA result layout each lane then owns ONE query and 4 keys of each
//     16-key tile, so row max / row sum are in-lane plus two cross-lane steps.
//   * The same per-lane scores, rounded to 16 bits, are exactly the B operand
//     of O^T = V^T P^T (16x16x32, contraction over 32 keys), so P never leaves
//     registers.  The V^T operand comes from the natural [key][dim] LDS tile
//     through ds_read_b64_tr_b16 (4 keys of one dim per lane per read).
//   * Exponentials are exp2 with scale*log2(e) folded into one FMA.
//   * For d = 40 the PV contraction pads d to 48; dim 40 of the V tile holds
//     1.0, so row 40 of O^T accumulates the row sum l on the matrix core.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef short s4v __attribute__((ext_vector_type(4)));
typedef short s8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef __bf16 b2v __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

struct F16 {
  static __device__ __forceinline__ f4v mma32(s8v a, s8v b, f4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f16v mma_32x32(s8v a, s8v b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
  }
  // two floats -> two fp16, round to nearest even
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, h2v));
  }
  static constexpr uint16_t kOne = 0x3C00;
  // A row sum of fp16-rounded P is within 2^-11 (relative) of the exact sum,
  // inside the 1e-3 bound on l, so the matrix-core ones-row sum may be reported.
  static constexpr bool kRoundedSumOk = true;
};

struct BF16 {
  static __device__ __forceinline__ f4v mma32(s8v a, s8v b, f4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8v, a), __builtin_bit_cast(b8v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f16v mma_32x32(s8v a, s8v b, f16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8v, a), __builtin_bit_cast(b8v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, b2v));
  }
  static constexpr uint16_t kOne = 0x3F80;
  // bf16 rounding (2^-8) is too coarse for a reported l: sum in fp32 as well.
  static constexpr bool kRoundedSumOk = false;
};

// Tuning knobs (compile-time).
#ifndef ATTN_FWD3
#define ATTN_FWD3 1        // 1: split-key forward kernel (32x32 scores, 8 waves per workgroup)
#endif
#ifndef ATTN_PINGPONG
#define ATTN_PINGPONG 0    // 1: the two key halves of a query group alternate MFMA and VALU phases
#endif
#ifndef ATTN_SWAP_ASM
#define ATTN_SWAP_ASM 0
#endif
#ifndef ATTN_PIPE
#define ATTN_PIPE 1        // 1: scores of block j+1 formed while block j's softmax runs
#endif
#ifndef ATTN_SGB
#define ATTN_SGB 1         // 1: hint the scheduler to spread MFMAs through the softmax
#endif
#ifndef ATTN_SGB_V
#define ATTN_SGB_V 4       // vector-ALU instructions between MFMAs in the interleave hint
#endif
#ifndef ATTN_MINW
#define ATTN_MINW 2        // minimum resident waves per SIMD the register budget must allow
#endif
#ifndef ATTN_QT
#define ATTN_QT 2          // 16-query tiles per wave in the forward kernels
#endif

constexpr int kWaves = 4;               // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kQT = ATTN_QT;            // 16-query tiles per wave (forward kernels)
constexpr int kQW = 16 * kQT;           // queries per wave
constexpr int kQWG = kWaves * kQW;      // queries per workgroup (forward kernels)

constexpr int kModeFlash = 0;    // online softmax, O only
constexpr int kModeFlashML = 1;  // online softmax, O and (m, l)
constexpr int kModePV = 2;       // softmax from given (m, l), O only

template <int D>
struct Shape {
  static constexpr int KS = D / 32;             // full K=32 MFMA steps over d
  static constexpr int KR = D % 32;             // remainder: 0, 8 or 16 dims, one zero-padded K=32 step
  // Lane group G of the remainder step holds dims [32 KS + 8 G, +8); groups
  // past the remainder get zeros in Q, and read K at a clamped, in-row offset
  // (finite data times zero).
  static constexpr int KRG = KR / 8;            // lane groups with real remainder dims
  static constexpr int MT = (D + 15) / 16;      // 16-row tiles of O^T
  static constexpr bool kOnes = (D % 16) != 0;  // V^T padding row D carries 1.0 -> l
  static constexpr int BN = D >= 160 ? 32 : 64; // keys per block
  // LDS row pitches in 16-bit elements, chosen so that the MFMA operand reads
  // are free of bank conflicts: K rows are read 16 consecutive rows at a time
  // (pitch = 4 * odd words); V is read by ds_read_b64_tr_b16 as 4 rows x 32 B
  // per 16 lanes (pitch mod 32 words in {8, 24}); the d = 40 V tile also
  // needs room for the padding columns 40..47.
  static constexpr int PK = D == 40 ? 40 : D + 8;
  static constexpr int PV = D == 40 ? 48 : (D == 80 ? 80 : D + 16);
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int NLD = (BN * CPR + kThreads - 1) / kThreads;
  static_assert(KR == 0 || KR == 8 || KR == 16, "head dim must be a multiple of 8 with remainder 0, 8 or 16 mod 32");
  static_assert(D >= 32, "head dim below 32 is not supported");
};

// Reductions over the four 16-lane groups (lanes li, li+16, li+32, li+48),
// which hold the same query in the MFMA result layout.  v_permlane16_swap
// exchanges the odd 16-lane rows of its first operand with the even rows of
// its second, and v_permlane32_swap the upper half of the first with the lower
// half of the second; with both operands equal to x, the two results together
// hold every row (half) once per lane.  The swaps are written as inline asm:
// this compiler's optimizer treats the two results of the swap builtins as
// interchangeable and folds a reduction over them away.  The leading s_nop
// covers the wait states a swap needs after a vector-ALU write of its inputs.
template <class Op>
__device__ __forceinline__ float group_reduce(float x, Op op) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 4\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  x = op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float group_max(float x) {
  return group_reduce(x, [](float a, float b) { return __builtin_fmaxf(a, b); });
}
__device__ __forceinline__ float group_sum(float x) {
  return group_reduce(x, [](float a, float b) { return a + b; });
}

// Offset (in elements) of lane group G's 8 dims in the remainder K step:
// clamped into the row so that groups without real dims read finite data.
template <int D>
__device__ __forceinline__ int rem_off(int G) {
  constexpr int KS = D / 32, KRG = (D % 32) / 8;
  return KS * 32 + (G < KRG ? G : KRG - 1) * 8;
}

// Empty asm that takes the packed probabilities as register inputs: they must
// be computed before this point in program order.
template <int A, int B>
__device__ __forceinline__ void pin(uint32_t (&pk)[A][B][4]) {
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int b = 0; b < B; ++b)
      asm volatile("" ::"v"(pk[a][b][0]), "v"(pk[a][b][1]), "v"(pk[a][b][2]), "v"(pk[a][b][3]));
}

// Scheduling hint for the current basic block: spread N matrix-core
// instructions evenly through the vector-ALU work instead of issuing them
// back to back (mask bits: 0x8 MFMA, 0x2 VALU, 0x100 LDS read).
template <int N>
__device__ __forceinline__ void interleave_mfma_valu() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    if (i % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Same for a block holding NDS LDS reads and NM matrix-core instructions:
// all reads first, then one MFMA every V vector-ALU instructions.
template <int NDS, int NM, int V>
__device__ __forceinline__ void interleave_reads_mfma_valu() {
  __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their no-wait maxima)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

// ---------------------------------------------------------------------------
// Forward kernel: FlashAttention (online softmax) or the PV pass of the
// partially fused softmax.  One workgroup = 4 waves = 128 queries of one head.
// K and V blocks of BN keys go through a ring of three LDS buffers shared by
// the waves.  The key loop is software pipelined: while the vector ALU turns
// the scores of block j into probabilities, the matrix cores already form the
// scores of block j+1; the product with V of block j follows, so both pipes
// have independent work in flight.  The last (possibly partial) block is
// peeled so that the steady-state loop carries no masking.
// ---------------------------------------------------------------------------
template <class TR, int D, int MODE>
struct Fwd {
  using S = Shape<D>;
  static constexpr int BN = S::BN, PK = S::PK, PV = S::PV, KS = S::KS, KR = S::KR, MT = S::MT;
  static constexpr int NKT = BN / 16, NKG = BN / 32, NBUF = ATTN_PIPE == 2 ? 4 : 3;
  // fp32 running sum on the vector ALU: needed when there is no ones row, or
  // when l is reported and the 16-bit P sum is not accurate enough for it.
  static constexpr bool kValuSum =
      MODE != kModePV && (!S::kOnes || (MODE == kModeFlashML && !TR::kRoundedSumOk));
  static constexpr int kSmem = NBUF * BN * (PK + PV);
  static constexpr int kQkMfma = NKT * (KS + (KR != 0 ? 1 : 0)) * kQT;  // MFMAs per block of Q K^T
  static constexpr int kPvMfma = NKG * MT * kQT;                          // MFMAs per block of P V
  static constexpr int kQkLds = NKT * (KS + (KR != 0 ? 1 : 0));           // LDS reads per block for K
  static constexpr int kPvLds = NKG * MT * 2;                             // LDS reads per block for V

  // S^T tile of the block in LDS at Kb: s[qt][kt][i] = q(query li of tile qt) . k(key 16 kt + 4 G + i)
  static __device__ __forceinline__ void qk(f4v (&s)[kQT][NKT], const uint16_t* Kb, const s8v (&qf)[kQT][KS],
                                            const s8v (&qr)[kQT], int G, int li) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const uint16_t* kr = Kb + (kt * 16 + li) * PK;
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) s[qt][kt] = (f4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const s8v a = *(const s8v*)(kr + ks * 32 + G * 8);
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) s[qt][kt] = TR::mma32(a, qf[qt][ks], s[qt][kt]);
      }
      if constexpr (KR != 0) {
        const s8v a = *(const s8v*)(kr + rem_off<D>(G));
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) s[qt][kt] = TR::mma32(a, qr[qt], s[qt][kt]);
      }
    }
  }

  // O^T += V^T P^T for the block in LDS at Vb.  Lane (G, li) supplies
  // V^T[dim 16 mt + li][keys 32 kg + 4 G + {0..3}] from the first transposing
  // read and keys 32 kg + 16 + 4 G + {0..3} from the second, which is the key
  // order of the packed P.
  static __device__ __forceinline__ void pv(f4v (&o)[kQT][MT], const uint16_t* Vb,
                                            const uint32_t (&pk)[kQT][NKG][4], int G, int li) {
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint16_t* va = Vb + (kg * 32 + G * 4 + (li >> 2)) * PV + mt * 16 + 4 * (li & 3);
        const s4v v0 = lds_read_tr16(va);
        const s4v v1 = lds_read_tr16(va + 16 * PV);
        const s8v vop = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) {
          const s8v pb = __builtin_bit_cast(s8v, (uint4){pk[qt][kg][0], pk[qt][kg][1], pk[qt][kg][2], pk[qt][kg][3]});
          o[qt][mt] = TR::mma32(vop, pb, o[qt][mt]);
        }
      }
    }
  }
};

template <class TR, int D, int MODE>
__global__ __launch_bounds__(kThreads, ATTN_MINW) void fwd_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ ml, int Nq, int Nk,
                                                          int qtiles, int nwg, float scale) {
  using F = Fwd<TR, D, MODE>;
  using S = typename F::S;
  constexpr int BN = F::BN, PK = F::PK, PV = F::PV, KS = F::KS, KR = F::KR, MT = F::MT;
  constexpr int NKT = F::NKT, NKG = F::NKG, NBUF = F::NBUF;
  constexpr bool kValuSum = F::kValuSum;
  __shared__ __attribute__((aligned(16))) uint16_t smem[F::kSmem];
  uint16_t* const kbase = smem;
  uint16_t* const vbase = smem + NBUF * BN * PK;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, G = lane >> 4, li = lane & 15;
  const float c = scale * kLog2e;

  const int tile = xcd_tile(nwg);
  const int head = tile / qtiles;
  const int qbase = (tile - head * qtiles) * kQWG + wave * kQW;
  const uint16_t* qh = q + (size_t)head * Nq * D;
  const uint16_t* kh = k + (size_t)head * Nk * D;
  const uint16_t* vh = v + (size_t)head * Nk * D;

  if constexpr (S::kOnes) {
    // padding columns D..PV-1 of every V buffer: 1.0 in column D, 0 elsewhere
    constexpr int PADC = PV - D;
    for (int e = tid; e < NBUF * BN * PADC; e += kThreads) {
      const int row = e / PADC, col = e - row * PADC;
      vbase[row * PV + D + col] = col == 0 ? TR::kOne : (uint16_t)0;
    }
  }

  // Q fragments (B operand of S^T = K Q^T): lane (G, li) holds query li of
  // each tile, dims [32 ks + 8 G, +8), and the zero-padded remainder dims.
  s8v qf[kQT][KS];
  s8v qr[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int row = qbase + qt * 16 + li;
    const bool ok = row < Nq;
    const uint16_t* qp = qh + (size_t)(ok ? row : 0) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s8v x = *(const s8v*)(qp + ks * 32 + G * 8);
      qf[qt][ks] = ok ? x : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
    }
    qr[qt] = (s8v){0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (KR != 0) {
      s8v x = *(const s8v*)(qp + rem_off<D>(G));
      qr[qt] = (ok && G < S::KRG) ? x : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // softmax state, per lane = per query of each tile; m in raw q.k units
  f4v o[kQT][MT];
  float m_used[kQT], m_true[kQT], lsum[kQT], mc[kQT], inv_l[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[qt][mt] = (f4v){0.f, 0.f, 0.f, 0.f};
    m_used[qt] = -INFINITY;
    m_true[qt] = -INFINITY;
    lsum[qt] = 0.f;
    mc[qt] = 0.f;
    inv_l[qt] = 1.f;
    if constexpr (MODE == kModePV) {
      const int row = qbase + qt * 16 + li;
      if (row < Nq) {
        const float2 st = *(const float2*)(ml + ((size_t)head * Nq + row) * 2);
        mc[qt] = st.x * kLog2e;  // m is stored in natural units of scale*q.k
        inv_l[qt] = 1.f / st.y;
      }
    }
  }

  // cooperative global -> register -> LDS staging of one K and V block
  uint4 kst[S::NLD], vst[S::NLD];
  auto gload = [&](int kb) {
    const int key0 = kb * BN;
#pragma unroll
    for (int r = 0; r < S::NLD; ++r) {
      const int ch = tid + r * kThreads;
      const int row = ch / S::CPR, col = (ch - row * S::CPR) * 8;
      const bool ok = ch < BN * S::CPR && key0 + row < Nk;
      const size_t off = (size_t)(ok ? key0 + row : 0) * D + (ok ? col : 0);
      uint4 kx = *(const uint4*)(kh + off);
      uint4 vx = *(const uint4*)(vh + off);
      kst[r] = ok ? kx : make_uint4(0, 0, 0, 0);
      vst[r] = ok ? vx : make_uint4(0, 0, 0, 0);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < S::NLD; ++r) {
      const int ch = tid + r * kThreads;
      if (ch < BN * S::CPR) {
        const int row = ch / S::CPR, col = (ch - row * S::CPR) * 8;
        *(uint4*)(kbase + buf * BN * PK + row * PK + col) = kst[r];
        *(uint4*)(vbase + buf * BN * PV + row * PV + col) = vst[r];
      }
    }
  };

  // Softmax of one block of scores into packed 16-bit P (and, for the online
  // form, the running max / lazy rescale).  Returns the per-tile rescale
  // factors to apply to O before this block's P V is added (1 if none).
  auto softmax = [&](f4v (&s)[kQT][NKT], uint32_t (&pk)[kQT][NKG][4], float (&alpha)[kQT]) -> bool {
    bool rescale = false;
    if constexpr (MODE != kModePV) {
      // Block max; the running reference max only moves when the block max
      // exceeds it by more than 2^8 in exp2 units, so exp2(s c - m c) <= 256
      // stays exact in 16-bit P and fp32 sums.  O / l does not depend on the
      // reference value, so this is still the exact softmax.
      bool need = false;
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) {
        float bm = s[qt][0][0];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) bm = __builtin_fmaxf(bm, s[qt][kt][i]);
        bm = group_max(bm);
        m_true[qt] = __builtin_fmaxf(m_true[qt], bm);
        need |= (bm - m_used[qt]) * c > 8.f;
      }
      rescale = __any(need);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) {
        const float mn = rescale ? m_true[qt] : m_used[qt];
        alpha[qt] = __builtin_amdgcn_exp2f((m_used[qt] - mn) * c);
        m_used[qt] = mn;
        mc[qt] = mn * c;
      }
    }
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      float ls = 0.f;
#pragma unroll
      for (int kg = 0; kg < NKG; ++kg) {
        float p[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p[h * 4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][2 * kg + h][i], c, -mc[qt]));
        if constexpr (kValuSum) {
#pragma unroll
          for (int j = 0; j < 8; ++j) ls += p[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[qt][kg][j] = TR::pack2(p[2 * j], p[2 * j + 1]);
      }
      if constexpr (kValuSum) lsum[qt] = lsum[qt] * (rescale ? alpha[qt] : 1.f) + ls;
    }
    return rescale;
  };
  auto apply_rescale = [&](const float (&alpha)[kQT]) {
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[qt][mt] *= alpha[qt];
  };

  const int nblk = (Nk + BN - 1) / BN;
  auto mask_tail = [&](f4v (&cur)[kQT][NKT]) {
    // keys past Nk (last block only) never contribute
    const int key0 = (nblk - 1) * BN;
    if (key0 + BN > Nk) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool dead = key0 + kt * 16 + G * 4 + i >= Nk;
#pragma unroll
          for (int qt = 0; qt < kQT; ++qt)
            if (dead) cur[qt][kt][i] = -INFINITY;
        }
    }
  };
  if constexpr (ATTN_PIPE == 2) {
    // Two-stage software pipeline over a ring of four LDS slots (block b in
    // slot b % 4).  Step j issues, as independent matrix-core work, the scores
    // of block j+1 and the product with V of block j-1, while the vector ALU
    // turns the scores of block j into probabilities; the rescale of O for
    // block j (rare) follows the product of block j-1 in program order.
    gload(0);
    swrite(0);
    if (nblk > 1) {
      gload(1);
      swrite(1);
    }
    wait_vmem_all();
    __syncthreads();
    f4v sa[kQT][NKT], sb[kQT][NKT];
    uint32_t pa[kQT][NKG][4], pb[kQT][NKG][4];
    F::qk(sa, kbase, qf, qr, G, li);
    if (nblk > 2) gload(2);
    auto kslot = [&](int b) { return kbase + (b & 3) * BN * PK; };
    auto vslot = [&](int b) { return vbase + (b & 3) * BN * PV; };
    auto advance = [&](int j) {
      if (j + 2 < nblk) swrite((j + 2) & 3);
      __syncthreads();
      if (j + 3 < nblk) gload(j + 3);
    };
    auto finish = [&](bool rescale, const float (&alpha)[kQT]) {
      if (MODE != kModePV && rescale) apply_rescale(alpha);
    };
    auto mid = [&](f4v (&cur)[kQT][NKT], f4v (&nxt)[kQT][NKT], uint32_t (&prev)[kQT][NKG][4],
                   uint32_t (&pcur)[kQT][NKG][4], int j) {
      float alpha[kQT];
      F::qk(nxt, kslot(j + 1), qf, qr, G, li);
      F::pv(o, vslot(j - 1), prev, G, li);
      const bool rescale = softmax(cur, pcur, alpha);
      if (ATTN_SGB)
        interleave_reads_mfma_valu<F::kQkLds + F::kPvLds, F::kQkMfma + F::kPvMfma, ATTN_SGB_V>();
      pin(pcur);
      finish(rescale, alpha);
      advance(j);
    };
    auto last = [&](f4v (&cur)[kQT][NKT], uint32_t (&prev)[kQT][NKG][4], uint32_t (&pcur)[kQT][NKG][4],
                    int j) {
      float alpha[kQT];
      F::pv(o, vslot(j - 1), prev, G, li);
      mask_tail(cur);
      const bool rescale = softmax(cur, pcur, alpha);
      finish(rescale, alpha);
      F::pv(o, vslot(j), pcur, G, li);
    };
    if (nblk == 1) {
      float alpha[kQT];
      mask_tail(sa);
      const bool rescale = softmax(sa, pa, alpha);
      finish(rescale, alpha);
      F::pv(o, vslot(0), pa, G, li);
    } else {
      {
        float alpha[kQT];
        F::qk(sb, kslot(1), qf, qr, G, li);
        const bool rescale = softmax(sa, pa, alpha);
        pin(pa);
        finish(rescale, alpha);
        advance(0);
      }
      for (int j = 1;;) {
        if (j == nblk - 1) {
          last(sb, pa, pb, j);
          break;
        }
        mid(sb, sa, pa, pb, j++);
        if (j == nblk - 1) {
          last(sa, pb, pa, j);
          break;
        }
        mid(sa, sb, pb, pa, j++);
      }
    }
  } else {
  // prologue: blocks 0 and 1 into LDS, scores of block 0, block 2 in flight
  gload(0);
  swrite(0);
  if (nblk > 1) {
    gload(1);
    swrite(1);
  }
  // All global loads issued so far (Q fragments, first blocks) are complete
  // here; saying so explicitly keeps the compiler from waiting on the
  // in-flight prefetch of later blocks inside the loop.
  wait_vmem_all();
  __syncthreads();
  f4v s[kQT][NKT];
  if (ATTN_PIPE) F::qk(s, kbase, qf, qr, G, li);
  if (nblk > 2) gload(2);

  // One step: O += V_j P_j for block j.  Pipelined form: the scores of block
  // j+1 go onto the matrix cores while the probabilities of block j are
  // formed; `cur` holds the scores of block j on entry and `nxt` receives
  // those of block j+1.
  int bk = ATTN_PIPE ? 1 : 0, bv = 0, bw = 2;  // ring slots of the K read, V(j), block j+2
  auto step = [&](f4v (&cur)[kQT][NKT], f4v (&nxt)[kQT][NKT], int j) {
    uint32_t pk[kQT][NKG][4];
    float alpha[kQT];
    if (ATTN_PIPE) {
      F::qk(nxt, kbase + bk * BN * PK, qf, qr, G, li);
    } else {
      F::qk(cur, kbase + bk * BN * PK, qf, qr, G, li);
    }
    const bool rescale = softmax(cur, pk, alpha);
    if (ATTN_SGB) interleave_mfma_valu<F::kQkMfma>();
    pin(pk);  // keep the exponentials ahead of the (rare) rescale branch
    if (MODE != kModePV && rescale) apply_rescale(alpha);
    F::pv(o, vbase + bv * BN * PV, pk, G, li);
    if (j + 2 < nblk) swrite(bw);
    __syncthreads();
    if (j + 3 < nblk) gload(j + 3);
    bk = bk == NBUF - 1 ? 0 : bk + 1;
    bv = bv == NBUF - 1 ? 0 : bv + 1;
    bw = bw == NBUF - 1 ? 0 : bw + 1;
  };
  // The last block (keys past Nk never contribute) closes the loop.
  auto last = [&](f4v (&cur)[kQT][NKT]) {
    if (!ATTN_PIPE) F::qk(cur, kbase + bk * BN * PK, qf, qr, G, li);
    const int key0 = (nblk - 1) * BN;
    if (key0 + BN > Nk) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool dead = key0 + kt * 16 + G * 4 + i >= Nk;
#pragma unroll
          for (int qt = 0; qt < kQT; ++qt)
            if (dead) cur[qt][kt][i] = -INFINITY;
        }
    }
    uint32_t pk[kQT][NKG][4];
    float alpha[kQT];
    const bool rescale = softmax(cur, pk, alpha);
    if (MODE != kModePV && rescale) apply_rescale(alpha);
    F::pv(o, vbase + bv * BN * PV, pk, G, li);
  };
  // unrolled by two so that the score registers swap roles instead of being copied
  f4v s2[kQT][NKT];
  for (int j = 0;;) {
    if (j + 1 >= nblk) {
      last(s);
      break;
    }
    step(s, s2, j++);
    if (j + 1 >= nblk) {
      last(s2);
      break;
    }
    step(s2, s, j++);
  }

  }

  // ---- epilogue: normalise, round, store
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int row = qbase + qt * 16 + li;
    float l = 0.f, l_report = 0.f;
    if constexpr (MODE != kModePV) {
      if constexpr (kValuSum) l_report = group_sum(lsum[qt]);
      if constexpr (S::kOnes) {
        // O^T row D = dim 16 (MT-1) + 4 G + i with G = (D % 16) / 4, i = D % 4;
        // O is normalised by the sum of the same rounded P it accumulated.
        constexpr int GL = (D % 16) / 4, IL = D % 4;
        l = __shfl(o[qt][MT - 1][IL], GL * 16 + li);
      } else {
        l = l_report;
      }
      if constexpr (!kValuSum) l_report = l;
    }
    const float inv = MODE == kModePV ? inv_l[qt] : 1.f / l;
    if (row < Nq) {
      uint16_t* op = out + ((size_t)head * Nq + row) * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int dim = mt * 16 + G * 4;
        if (dim < D) {
          uint2 w;
          w.x = TR::pack2(o[qt][mt][0] * inv, o[qt][mt][1] * inv);
          w.y = TR::pack2(o[qt][mt][2] * inv, o[qt][mt][3] * inv);
          *(uint2*)(op + dim) = w;
        }
      }
      if constexpr (MODE == kModeFlashML) {
        if (G == 0) {
          // l was accumulated against m_used; report it against the true max
          const float lt = l_report * __builtin_amdgcn_exp2f((m_used[qt] - m_true[qt]) * c);
          *(float2*)(ml + ((size_t)head * Nq + row) * 2) = make_float2(m_true[qt] * scale, lt);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Forward kernel, split-key form: FlashAttention (online softmax) or the PV
// pass of the partially fused softmax.
//
// One workgroup = 8 waves = 4 query groups of 32 queries x 2 key halves; the
// two waves of a query group walk alternate 32-key blocks (the key range is
// split in two, as in the block-split reduction) and merge their partial
// (m, l, O) through LDS at the end.  Eight waves per workgroup put four
// waves on each SIMD, so one wave's matrix-core work overlaps another's
// softmax arithmetic.
//
//   * S^T = K Q^T on 32x32x16 MFMAs: a 32-key x 32-query tile per block, the
//     head dim in K=16 steps (d = 40 pads to 48).  Lane l owns query l % 32
//     and 16 of the 32 keys; lanes l and l ^ 32 share a query.
//   * P is rounded to 16 bits, and one v_permlane16_swap per pair of packed
//     registers turns the 32x32 result layout into the B operands of two
//     16x16x32 MFMAs (queries 0-15 and 16-31) for O^T += V^T P^T.  V^T comes
//     from the [key][dim] LDS tile through ds_read_b64_tr_b16, in the key
//     order the swap produces.
//   * d = 40 pads the PV product to 48 rows; LDS column 40 of V holds 1.0 so
//     row 40 of O^T is the row sum l of the same rounded P.
// ---------------------------------------------------------------------------
constexpr int kW3 = 8;              // waves per workgroup
constexpr int kT3 = 64 * kW3;       // threads per workgroup
constexpr int kQ3 = 32;             // queries per wave
constexpr int kQWG3 = 4 * kQ3;      // queries per workgroup
constexpr int kBN3 = 32;            // keys per block

template <int D>
struct Shape3 {
  static constexpr int KS = (D + 15) / 16;      // K=16 steps of Q K^T (last one zero padded for d = 40)
  static constexpr int MT = (D + 15) / 16;      // 16-row tiles of O^T
  static constexpr bool kOnes = (D % 16) != 0;  // LDS column D of V holds 1.0 -> O^T row D = l
  // LDS row pitches (16-bit elements): K rows are read 32 consecutive rows at
  // a time (pitch = 4 * odd words); V is read by ds_read_b64_tr_b16 as 4 rows
  // x 32 bytes per 16 lanes (pitch mod 32 words in {8, 24}).
  static constexpr int PK = D == 40 ? 40 : D + 8;
  static constexpr int PV = D == 40 ? 48 : (D == 80 ? 80 : D + 16);
  static constexpr int NBUF = D >= 160 ? 2 : 3;  // ring slots per key half
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int NLD = (kBN3 * CPR + 255) / 256;
  static constexpr int SLOT = kBN3 * (PK + PV);  // 16-bit elements per slot (K then V)
  static constexpr int NEX = 2 * MT * 4 + 8;     // floats per lane handed over in the merge
  static constexpr int RING = 2 * NBUF * SLOT;   // 16-bit elements, both halves
  static constexpr int SMEM = RING > NEX * 256 * 2 ? RING : NEX * 256 * 2;
};

// 16-lane-row exchange: returns (A.row0, B.row0, A.row2, B.row2) in a and
// (A.row1, B.row1, A.row3, B.row3) in b.  The operands here are distinct
// values, so the builtin is safe from the fold described above and lets the
// compiler place the required wait states itself.
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
#if ATTN_SWAP_ASM
  asm volatile("s_nop 4\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
#else
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
#endif
}
// max / sum over lanes l and l ^ 32
__device__ __forceinline__ float pair_max32(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return __builtin_fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float pair_sum32(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

template <class TR, int D, int MODE>
__global__ __launch_bounds__(kT3) void fwd3_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   uint16_t* __restrict__ out,
                                                   float* __restrict__ ml, int Nq, int Nk,
                                                   int qtiles, int nwg, float scale) {
  using S = Shape3<D>;
  constexpr int KS = S::KS, MT = S::MT, PK = S::PK, PV = S::PV, NBUF = S::NBUF, NEX = S::NEX;
  constexpr bool kValuSum = MODE != kModePV && (!S::kOnes || (MODE == kModeFlashML && !TR::kRoundedSumOk));
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::SMEM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int qg = wave & 3, half = wave >> 2, htid = tid & 255;
  const int l32 = lane & 31, hi = lane >> 5;  // 32x32 layout: query l32, key subgroup hi
  const int G = lane >> 4, li = lane & 15;    // 16x16 layout
  const float c = scale * kLog2e;

  const int tile = xcd_tile(nwg);
  const int head = tile / qtiles;
  const int qbase = (tile - head * qtiles) * kQWG3 + qg * kQ3;
  const uint16_t* qh = q + (size_t)head * Nq * D;
  const uint16_t* kh = k + (size_t)head * Nk * D;
  const uint16_t* vh = v + (size_t)head * Nk * D;
  uint16_t* const ring = smem + half * NBUF * S::SLOT;

  if constexpr (S::kOnes) {
    // padding columns D..PV-1 of every V slot of this half: 1.0 in column D, 0 elsewhere
    constexpr int PADC = PV - D;
    for (int e = htid; e < NBUF * kBN3 * PADC; e += 256) {
      const int r = e / PADC, col = e - r * PADC;
      ring[(r / kBN3) * S::SLOT + kBN3 * PK + (r % kBN3) * PV + D + col] = col == 0 ? TR::kOne : (uint16_t)0;
    }
  }

  // Q operand (B of the 32x32x16 MFMA): query l32, dims [16 ks + 8 hi, +8); zero past d.
  s8v qf[KS];
  {
    const int row = qbase + l32;
    const bool ok = row < Nq;
    const uint16_t* qp = qh + (size_t)(ok ? row : 0) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 16 + hi * 8;
      s8v x = *(const s8v*)(qp + (d0 < D ? d0 : D - 8));
      qf[ks] = (ok && d0 < D) ? x : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // state: m in raw q.k units, in the 32x32 layout (query l32); O in the 16x16 layout
  f4v o[2][MT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[qt][mt] = (f4v){0.f, 0.f, 0.f, 0.f};
  float m_used = -INFINITY, m_true = -INFINITY, lsum = 0.f, mc = 0.f;
  if constexpr (MODE == kModePV) {
    const int row = qbase + l32;
    if (row < Nq) mc = ml[((size_t)head * Nq + row) * 2] * kLog2e;  // m is stored in natural units
  }

  const int nblk = (Nk + kBN3 - 1) / kBN3;
  const int niter = (nblk + 1) / 2;
  // staging of this half's block for iteration `it` (key block 2 it + half)
  uint4 kst[S::NLD], vst[S::NLD];
  auto gload = [&](int it) {
    const int key0 = (2 * it + half) * kBN3;
#pragma unroll
    for (int r = 0; r < S::NLD; ++r) {
      const int ch = htid + r * 256;
      const int row = ch / S::CPR, col = (ch - row * S::CPR) * 8;
      const bool ok = ch < kBN3 * S::CPR && key0 + row < Nk;
      const size_t off = (size_t)(ok ? key0 + row : 0) * D + (ok ? col : 0);
      uint4 kx = *(const uint4*)(kh + off);
      uint4 vx = *(const uint4*)(vh + off);
      kst[r] = ok ? kx : make_uint4(0, 0, 0, 0);
      vst[r] = ok ? vx : make_uint4(0, 0, 0, 0);
    }
  };
  auto swrite = [&](int slot) {
    uint16_t* ks_ = ring + slot * S::SLOT;
    uint16_t* vs_ = ks_ + kBN3 * PK;
#pragma unroll
    for (int r = 0; r < S::NLD; ++r) {
      const int ch = htid + r * 256;
      if (ch < kBN3 * S::CPR) {
        const int row = ch / S::CPR, col = (ch - row * S::CPR) * 8;
        *(uint4*)(ks_ + row * PK + col) = kst[r];
        *(uint4*)(vs_ + row * PV + col) = vst[r];
      }
    }
  };

  // key order after the row swap: lane group G holds keys vbase_g + {0..3} and vbase_g + 8 + {0..3}
  const int vbase_g = (G & 1) * 16 + (G >> 1) * 4;

  // ---- S^T of one 32-key block (matrix cores)
  auto qk_block = [&](const uint16_t* Ks) {
    f16v sc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 16 + hi * 8;
      const s8v a = *(const s8v*)(Ks + l32 * PK + (d0 < D ? d0 : D - 8));
      sc = TR::mma_32x32(a, qf[ks], sc);
    }
    return sc;
  };
  // ---- probabilities of one block (vector ALU): mask, running max, lazy
  // rescale of O, exp2, rounding to 16 bits and the row swap into the two
  // 16x16x32 B operands (queries 0-15 and 16-31)
  auto soft_block = [&](f16v sc, int kb, s8v& P0, s8v& P1) {
    if (kb * kBN3 + kBN3 > Nk) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * kBN3 + (i / 4) * 8 + hi * 4 + (i % 4) >= Nk) sc[i] = -INFINITY;
    }
    if constexpr (MODE != kModePV) {
      float bm = sc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) bm = __builtin_fmaxf(bm, sc[i]);
      bm = pair_max32(bm);
      m_true = __builtin_fmaxf(m_true, bm);
      // lazy rescale: the reference max moves only when the block max exceeds
      // it by more than 2^8 in exp2 units; O / l is independent of it.
      if (__any((bm - m_used) * c > 8.f)) {
        const float alpha = __builtin_amdgcn_exp2f((m_used - m_true) * c);
        m_used = m_true;
        mc = m_used * c;
        lsum *= alpha;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const float ao = __shfl(alpha, qt * 16 + li);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) o[qt][mt] *= ao;
        }
      }
    }
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c, -mc));
    if constexpr (kValuSum) {
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) ls += p[i];
      lsum += ls;
    }
    uint32_t pa[4], pb[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      pa[d] = TR::pack2(p[2 * d], p[2 * d + 1]);
      pb[d] = TR::pack2(p[8 + 2 * d], p[8 + 2 * d + 1]);
      swap16(pa[d], pb[d]);  // pa: queries 0-15, pb: queries 16-31
    }
    P0 = __builtin_bit_cast(s8v, (uint4){pa[0], pa[1], pa[2], pa[3]});
    P1 = __builtin_bit_cast(s8v, (uint4){pb[0], pb[1], pb[2], pb[3]});
  };
  // ---- O^T += V^T P^T for one block (matrix cores)
  auto pv_block = [&](const uint16_t* Vs, const s8v& P0, const s8v& P1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint16_t* va = Vs + (vbase_g + (li >> 2)) * PV + mt * 16 + 4 * (li & 3);
      const s4v v0 = lds_read_tr16(va);
      const s4v v1 = lds_read_tr16(va + 8 * PV);
      const s8v vop = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      o[0][mt] = TR::mma32(vop, P0, o[0][mt]);
      o[1][mt] = TR::mma32(vop, P1, o[1][mt]);
    }
  };
  auto kslot = [&](int b) { return ring + (b % NBUF) * S::SLOT; };

  if constexpr (ATTN_PINGPONG) {
    // Ping-pong: the two waves of a query group share a SIMD and run
    // opposite phases between workgroup barriers -- one issues matrix-core
    // work (scores of its block b, product with V of block b-1) while the
    // other forms the probabilities of its current block.  Half 0 is one
    // phase ahead of half 1.  This half's block b is key block 2 b + half.
    const int nb = (nblk - half + 1) / 2;
    // prologue: blocks 0 and 1 of each half into slots 0 and 1; block 2 in flight
#pragma unroll
    for (int d = 0; d + 1 < NBUF; ++d) {
      if (d < nb) {
        gload(d);
        swrite(d % NBUF);
      }
    }
    wait_vmem_all();
    __syncthreads();
    if (NBUF - 1 < nb) gload(NBUF - 1);
    f16v sc = {};
    s8v P0 = {}, P1 = {};
    const int T = 2 * niter + 2;
    for (int t = 0; t < T; ++t) {
      if (((t + half) & 1) == 0) {
        const int b = (t - half) >> 1;  // matrix-core phase of block b
        if (b < nb) sc = qk_block(kslot(b));
        if (b >= 1 && b - 1 < nb) pv_block(kslot(b - 1) + kBN3 * PK, P0, P1);
      } else {
        const int b = (t - 1 - half) >> 1;  // vector-ALU phase of block b
        if (b >= 0 && b < nb) {
          soft_block(sc, 2 * b + half, P0, P1);
          // staging: block b+NBUF-1 into the slot block b-1 has left, next block in flight
          if (b + NBUF - 1 < nb) swrite((b + NBUF - 1) % NBUF);
          if (b + NBUF < nb) gload(b + NBUF);
        }
      }
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int d = 0; d + 1 < NBUF; ++d) {
      if (d < niter) {
        gload(d);
        swrite(d);
      }
    }
    wait_vmem_all();
    __syncthreads();
    if (NBUF - 1 < niter) gload(NBUF - 1);
    for (int it = 0; it < niter; ++it) {
      const int kb = 2 * it + half;
      if (kb < nblk) {
        s8v P0, P1;
        soft_block(qk_block(kslot(it)), kb, P0, P1);
        pv_block(kslot(it) + kBN3 * PK, P0, P1);
      }
      if (it + NBUF - 1 < niter) swrite((it + NBUF - 1) % NBUF);
      __syncthreads();
      if (it + NBUF < niter) gload(it + NBUF);
    }
  }

  // ---- per-query state in the 16x16 layout: lane (G, li) <- query qt*16 + li
  float mo[2], mto[2], lo[2], lro[2];
  const float lfull = kValuSum ? pair_sum32(lsum) : 0.f;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    mo[qt] = __shfl(m_used, qt * 16 + li);
    mto[qt] = __shfl(m_true, qt * 16 + li);
    if constexpr (MODE == kModePV) {
      lo[qt] = 0.f;
      lro[qt] = 0.f;
    } else {
      if constexpr (S::kOnes) {
        constexpr int GL = (D % 16) / 4, IL = D % 4;
        lo[qt] = __shfl(o[qt][MT - 1][IL], GL * 16 + li);
      } else {
        lo[qt] = __shfl(lfull, qt * 16 + li);
      }
      lro[qt] = kValuSum ? __shfl(lfull, qt * 16 + li) : lo[qt];
    }
  }

  // ---- merge the two key halves: half 1 hands its state to half 0 through LDS
  float* ex = (float*)smem + qg * NEX * 64 + lane;
  if (half == 1) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) ex[((qt * MT + mt) * 4 + i) * 64] = o[qt][mt][i];
      ex[(2 * MT * 4 + qt * 4 + 0) * 64] = mo[qt];
      ex[(2 * MT * 4 + qt * 4 + 1) * 64] = mto[qt];
      ex[(2 * MT * 4 + qt * 4 + 2) * 64] = lo[qt];
      ex[(2 * MT * 4 + qt * 4 + 3) * 64] = lro[qt];
    }
  }
  __syncthreads();
  if (half == 1) return;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float mB = ex[(2 * MT * 4 + qt * 4 + 0) * 64];
    const float mtB = ex[(2 * MT * 4 + qt * 4 + 1) * 64];
    const float lB = ex[(2 * MT * 4 + qt * 4 + 2) * 64];
    const float lrB = ex[(2 * MT * 4 + qt * 4 + 3) * 64];
    float fA = 1.f, fB = 1.f, M = mo[qt];
    if constexpr (MODE != kModePV) {
      // a half that saw no key holds (-inf, 0, 0) and contributes nothing
      M = __builtin_fmaxf(mo[qt], mB);
      fA = __builtin_amdgcn_exp2f((mo[qt] - M) * c);
      fB = __builtin_amdgcn_exp2f((mB - M) * c);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[qt][mt][i] = o[qt][mt][i] * fA + ex[((qt * MT + mt) * 4 + i) * 64] * fB;
    const float l = lo[qt] * fA + lB * fB;
    const float lr = lro[qt] * fA + lrB * fB;
    const float mt_all = __builtin_fmaxf(mto[qt], mtB);
    const int row = qbase + qt * 16 + li;
    float inv;
    if constexpr (MODE == kModePV) {
      inv = row < Nq ? 1.f / ml[((size_t)head * Nq + row) * 2 + 1] : 0.f;
    } else {
      inv = 1.f / l;
    }
    if (row < Nq) {
      uint16_t* op = out + ((size_t)head * Nq + row) * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int dim = mt * 16 + G * 4;
        if (dim < D) {
          uint2 w;
          w.x = TR::pack2(o[qt][mt][0] * inv, o[qt][mt][1] * inv);
          w.y = TR::pack2(o[qt][mt][2] * inv, o[qt][mt][3] * inv);
          *(uint2*)(op + dim) = w;
        }
      }
      if constexpr (MODE == kModeFlashML) {
        if (G == 0) {
          // l was accumulated against the reference max M; report it against the true max
          const float lt = lr * __builtin_amdgcn_exp2f((M - mt_all) * c);
          *(float2*)(ml + ((size_t)head * Nq + row) * 2) = make_float2(mt_all * scale, lt);
        }
      }
    }
  }
}

template <class TR, int D, int MODE>
hipError_t launch_fwd3_t(const Problem& p) {
  const int qtiles = (p.Nq + kQWG3 - 1) / kQWG3;
  const long long nwg = (long long)p.BH * qtiles;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd3_kernel<TR, D, MODE>), dim3((unsigned)nwg), dim3(kT3), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v, (uint16_t*)p.out,
                     p.ml, p.Nq, p.Nk, qtiles, (int)nwg, p.scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stats kernel (partially fused softmax, pass 1).  One workgroup = 4 waves on
// the same 64 queries of one head.  The row of A for each query is cut into
// key blocks of 32; wave w reduces blocks w, w+4, w+8, ... to a running
// (max, sum of exp) pair, and the four partial pairs are merged through LDS
// with (m,l)+(m',l') = (M, l e^(m-M) + l' e^(m'-M)) before the single store.
// K is read straight from global memory (L2) into MFMA operand registers.
// ---------------------------------------------------------------------------
constexpr int kSQT = 4;              // 16-query tiles per workgroup
constexpr int kSQ = 16 * kSQT;       // queries per workgroup (stats kernel)
constexpr int kSBN = 32;             // keys per block (stats kernel)

template <class TR, int D>
__global__ __launch_bounds__(kThreads) void stats_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         float* __restrict__ ml, int Nq, int Nk,
                                                         int qtiles, int nwg, float scale) {
  using S = Shape<D>;
  constexpr int KS = S::KS, KR = S::KR;
  constexpr int NKT = kSBN / 16;
  __shared__ float part_m[kWaves][kSQ];
  __shared__ float part_l[kWaves][kSQ];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, G = lane >> 4, li = lane & 15;
  const float c = scale * kLog2e;

  const int tile = xcd_tile(nwg);
  const int head = tile / qtiles;
  const int qbase = (tile - head * qtiles) * kSQ;
  const uint16_t* qh = q + (size_t)head * Nq * D;
  const uint16_t* kh = k + (size_t)head * Nk * D;

  s8v qf[kSQT][KS > 0 ? KS : 1];
  s8v qr[kSQT];
#pragma unroll
  for (int qt = 0; qt < kSQT; ++qt) {
    const int row = qbase + qt * 16 + li;
    const bool ok = row < Nq;
    const uint16_t* qp = qh + (size_t)(ok ? row : 0) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s8v x = *(const s8v*)(qp + ks * 32 + G * 8);
      qf[qt][ks] = ok ? x : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
    }
    if constexpr (KR != 0) {
      s8v x = *(const s8v*)(qp + rem_off<D>(G));
      qr[qt] = (ok && G < S::KRG) ? x : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  float m[kSQT], l[kSQT];
#pragma unroll
  for (int qt = 0; qt < kSQT; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.f;
  }

  // K operand registers for one block: lane (G, li) holds key 16 kt + li,
  // dims [32 ks + 8 G, +8) and the remainder dims.
  s8v ka[NKT][KS > 0 ? KS : 1];
  s8v kr8[NKT];
  auto kload = [&](int kb) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const int key = kb * kSBN + kt * 16 + li;
      const bool ok = key < Nk;
      const uint16_t* kp = kh + (size_t)(ok ? key : 0) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s8v x = *(const s8v*)(kp + ks * 32 + G * 8);
        ka[kt][ks] = ok ? x : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
      }
      if constexpr (KR != 0) {
        s8v x = *(const s8v*)(kp + rem_off<D>(G));
        kr8[kt] = ok ? x : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  };

  const int nblk = (Nk + kSBN - 1) / kSBN;
  for (int kb = wave; kb < nblk; kb += kWaves) {
    kload(kb);
#pragma unroll
    for (int qt = 0; qt < kSQT; ++qt) {
      f4v s[NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        s[kt] = (f4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[kt] = TR::mma32(ka[kt][ks], qf[qt][ks], s[kt]);
        if constexpr (KR != 0) s[kt] = TR::mma32(kr8[kt], qr[qt], s[kt]);
      }
      if (kb * kSBN + kSBN > Nk) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb * kSBN + kt * 16 + G * 4 + i >= Nk) s[kt][i] = -INFINITY;
      }
      // block partial (bm, bl) merged into the running pair
      float bm = s[0][0];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bm = __builtin_fmaxf(bm, s[kt][i]);
      bm = group_max(bm);
      const float mn = __builtin_fmaxf(m[qt], bm);
      const float mnc = mn * c;
      float bl = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bl += __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], c, -mnc));
      l[qt] = l[qt] * __builtin_amdgcn_exp2f((m[qt] - mn) * c) + bl;
      m[qt] = mn;
    }
  }

  // per-wave partial pairs: the four lane groups hold disjoint keys of the same query
#pragma unroll
  for (int qt = 0; qt < kSQT; ++qt) {
    const float lw = group_sum(l[qt]);
    if (G == 0) {
      part_m[wave][qt * 16 + li] = m[qt];
      part_l[wave][qt * 16 + li] = lw;
    }
  }
  __syncthreads();
  if (tid < kSQ) {
    const int row = qbase + tid;
    float M = part_m[0][tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = __builtin_fmaxf(M, part_m[w][tid]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float pm = part_m[w][tid];
      // a wave that saw no key of this row holds (-inf, 0) and adds nothing
      if (pm != -INFINITY) L += part_l[w][tid] * __builtin_amdgcn_exp2f((pm - M) * c);
    }
    if (row < Nq) *(float2*)(ml + ((size_t)head * Nq + row) * 2) = make_float2(M * scale, L);
  }
}

template <class TR, int D, int MODE>
hipError_t launch_fwd_t(const Problem& p) {
  const int qtiles = (p.Nq + kQWG - 1) / kQWG;
  const long long nwg = (long long)p.BH * qtiles;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_kernel<TR, D, MODE>), dim3((unsigned)nwg), dim3(kThreads), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v, (uint16_t*)p.out,
                     p.ml, p.Nq, p.Nk, qtiles, (int)nwg, p.scale);
  return hipGetLastError();
}

template <class TR, int D>
hipError_t launch_stats_t(const Problem& p) {
  const int qtiles = (p.Nq + kSQ - 1) / kSQ;
  const long long nwg = (long long)p.BH * qtiles;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((stats_kernel<TR, D>), dim3((unsigned)nwg), dim3(kThreads), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, p.ml, p.Nq, p.Nk, qtiles, (int)nwg,
                     p.scale);
  return hipGetLastError();
}

template <template <class, int> class L, class TR>
hipError_t by_dim(const Problem& p) {
  switch (p.d) {
    case 40: return L<TR, 40>::run(p);
    case 80: return L<TR, 80>::run(p);
    case 160: return L<TR, 160>::run(p);
    default: return hipErrorInvalidValue;
  }
}
template <template <class, int> class L>
hipError_t by_type(const Problem& p) {
  return p.dt == ATTN_BF16 ? by_dim<L, BF16>(p) : by_dim<L, F16>(p);
}

template <class TR, int D> struct StatsL { static hipError_t run(const Problem& p) { return launch_stats_t<TR, D>(p); } };
template <class TR, int D> struct PvL {
  static hipError_t run(const Problem& p) {
    return ATTN_FWD3 ? launch_fwd3_t<TR, D, kModePV>(p) : launch_fwd_t<TR, D, kModePV>(p);
  }
};
template <class TR, int D> struct FlashL {
  static hipError_t run(const Problem& p) {
    if (ATTN_FWD3) return p.ml ? launch_fwd3_t<TR, D, kModeFlashML>(p) : launch_fwd3_t<TR, D, kModeFlash>(p);
    return p.ml ? launch_fwd_t<TR, D, kModeFlashML>(p) : launch_fwd_t<TR, D, kModeFlash>(p);
  }
};

}  // namespace

hipError_t launch_mfma_stats(const Problem& p) { return by_type<StatsL>(p); }
hipError_t launch_mfma_pv(const Problem& p) { return by_type<PvL>(p); }
hipError_t launch_mfma_flash(const Problem& p) { return by_type<FlashL>(p); }

}  // namespace attn
