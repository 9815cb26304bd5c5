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
//   * Scores are formed transposed, S^T = K Q^T, with the 16x16x32 MFMA
//     (plus one 16x16x16 step for a head-dim remainder of 8 or 16).  In the
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
  static __device__ __forceinline__ f4v mma16(s4v a, s4v b, f4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4v, a), __builtin_bit_cast(h4v, b), c, 0, 0, 0);
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
  static __device__ __forceinline__ f4v mma16(s4v a, s4v b, f4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, b2v));
  }
  static constexpr uint16_t kOne = 0x3F80;
  // bf16 rounding (2^-8) is too coarse for a reported l: sum in fp32 as well.
  static constexpr bool kRoundedSumOk = false;
};

constexpr int kWaves = 4;               // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kQT = 2;                  // 16-query tiles per wave (forward kernels)
constexpr int kQW = 16 * kQT;           // queries per wave
constexpr int kQWG = kWaves * kQW;      // queries per workgroup (forward kernels)

constexpr int kModeFlash = 0;    // online softmax, O only
constexpr int kModeFlashML = 1;  // online softmax, O and (m, l)
constexpr int kModePV = 2;       // softmax from given (m, l), O only

template <int D>
struct Shape {
  static constexpr int KS = D / 32;             // full K=32 MFMA steps over d
  static constexpr int KR = D % 32;             // remainder step: 0, 8 (padded to 16) or 16
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
};

__device__ __forceinline__ float wave_max_xor_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum_xor_16_32(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
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

// ---------------------------------------------------------------------------
// Forward kernel: FlashAttention (online softmax) or the PV pass of the
// partially fused softmax.  One workgroup = 4 waves = 128 queries of one head;
// K and V blocks are staged in LDS (double buffered) and shared by the waves.
// ---------------------------------------------------------------------------
template <class TR, int D, int MODE>
__global__ __launch_bounds__(kThreads) void fwd_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ ml, int Nq, int Nk,
                                                       int qtiles, int nwg, float scale) {
  using S = Shape<D>;
  constexpr int BN = S::BN, PK = S::PK, PV = S::PV, KS = S::KS, KR = S::KR, MT = S::MT;
  constexpr int NKT = BN / 16, NKG = BN / 32;
  // fp32 running sum on the vector ALU: needed when there is no ones row, or
  // when l is reported and the 16-bit P sum is not accurate enough for it.
  constexpr bool kValuSum = MODE != kModePV && (!S::kOnes || (MODE == kModeFlashML && !TR::kRoundedSumOk));
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BN * (PK + PV)];
  uint16_t* const kbuf0 = smem;
  uint16_t* const vbuf0 = smem + 2 * BN * PK;

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
    // padding columns D..PV-1 of both V buffers: 1.0 in column D, 0 elsewhere
    constexpr int PADC = PV - D;
    for (int e = tid; e < 2 * BN * PADC; e += kThreads) {
      const int row = e / PADC, col = e - row * PADC;
      vbuf0[row * PV + D + col] = col == 0 ? TR::kOne : (uint16_t)0;
    }
  }

  // Q fragments (B operand of S^T = K Q^T): lane (G, li) holds query li of
  // each tile, dims [32 ks + 8 G, +8) and the remainder dims [32 KS + 4 G, +4).
  s8v qf[kQT][KS > 0 ? KS : 1];
  s4v qr[kQT];
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
    if constexpr (KR == 8) {
      s4v x = *(const s4v*)(qp + KS * 32 + (G & 1) * 4);
      qr[qt] = (ok && G < 2) ? x : (s4v){0, 0, 0, 0};
    } else if constexpr (KR == 16) {
      s4v x = *(const s4v*)(qp + KS * 32 + G * 4);
      qr[qt] = ok ? x : (s4v){0, 0, 0, 0};
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
        *(uint4*)(kbuf0 + buf * BN * PK + row * PK + col) = kst[r];
        *(uint4*)(vbuf0 + buf * BN * PV + row * PV + col) = vst[r];
      }
    }
  };

  const int nblk = (Nk + BN - 1) / BN;
  gload(0);
  swrite(0);
  __syncthreads();

  for (int kb = 0; kb < nblk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nblk) gload(kb + 1);
    const uint16_t* Kb = kbuf0 + buf * BN * PK;
    const uint16_t* Vb = vbuf0 + buf * BN * PV;

    // ---- S^T = K Q^T for the block: s[qt][kt][i] = q(query li) . k(key kb*BN + 16 kt + 4 G + i)
    f4v s[kQT][NKT];
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
        s4v a = *(const s4v*)(kr + KS * 32 + (KR == 8 ? (G & 1) * 4 : G * 4));
        if (KR == 8 && G >= 2) a = (s4v){0, 0, 0, 0};
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) s[qt][kt] = TR::mma16(a, qr[qt], s[qt][kt]);
      }
    }
    // keys past Nk (last block only) never contribute
    if (kb * BN + BN > Nk) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool dead = kb * BN + kt * 16 + G * 4 + i >= Nk;
#pragma unroll
          for (int qt = 0; qt < kQT; ++qt)
            if (dead) s[qt][kt][i] = -INFINITY;
        }
    }

    if constexpr (MODE != kModePV) {
      // ---- online softmax: block max, lazy rescale of the running state.
      // The running reference max only moves when the block max exceeds it by
      // more than 2^8 in exp2 units; until then exp2(s c - m c) <= 256, which
      // fp16 P and the fp32 sums hold exactly as well.  The final O / l is the
      // same for any reference value, so this is still the exact softmax.
      bool need = false;
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) {
        float bm = s[qt][0][0];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) bm = fmaxf(bm, s[qt][kt][i]);
        bm = wave_max_xor_16_32(bm);
        m_true[qt] = fmaxf(m_true[qt], bm);
        need |= (bm - m_used[qt]) * c > 8.f;
      }
      if (__any(need)) {
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) {
          const float mn = m_true[qt];
          const float alpha = __builtin_amdgcn_exp2f((m_used[qt] - mn) * c);
          m_used[qt] = mn;
          mc[qt] = mn * c;
          lsum[qt] *= alpha;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) o[qt][mt] *= alpha;
        }
      }
    }

    // ---- P = exp2(s c - m c), rounded to 16 bits, packed as the B operand of O^T += V^T P^T
    uint32_t pk[kQT][NKG][4];
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
      if constexpr (kValuSum) lsum[qt] += ls;
    }

    // ---- O^T += V^T P^T.  Lane (G, li) supplies V^T[dim 16 mt + li][keys 32 kg + 4 G + {0..3}]
    // from the first read and keys 32 kg + 16 + 4 G + {0..3} from the second,
    // matching the key order of the packed P above.
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

    if (kb + 1 < nblk) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, round, store
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int row = qbase + qt * 16 + li;
    float l = 0.f, l_report = 0.f;
    if constexpr (MODE != kModePV) {
      if constexpr (kValuSum) l_report = wave_sum_xor_16_32(lsum[qt]);
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
  s4v qr[kSQT];
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
    if constexpr (KR == 8) {
      s4v x = *(const s4v*)(qp + KS * 32 + (G & 1) * 4);
      qr[qt] = (ok && G < 2) ? x : (s4v){0, 0, 0, 0};
    } else if constexpr (KR == 16) {
      s4v x = *(const s4v*)(qp + KS * 32 + G * 4);
      qr[qt] = ok ? x : (s4v){0, 0, 0, 0};
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
  s4v kr4[NKT];
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
      if constexpr (KR == 8) {
        s4v x = *(const s4v*)(kp + KS * 32 + (G & 1) * 4);
        kr4[kt] = (ok && G < 2) ? x : (s4v){0, 0, 0, 0};
      } else if constexpr (KR == 16) {
        s4v x = *(const s4v*)(kp + KS * 32 + G * 4);
        kr4[kt] = ok ? x : (s4v){0, 0, 0, 0};
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
        if constexpr (KR != 0) s[kt] = TR::mma16(kr4[kt], qr[qt], s[kt]);
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
        for (int i = 0; i < 4; ++i) bm = fmaxf(bm, s[kt][i]);
      bm = wave_max_xor_16_32(bm);
      const float mn = fmaxf(m[qt], bm);
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
    const float lw = wave_sum_xor_16_32(l[qt]);
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
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, part_m[w][tid]);
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
template <class TR, int D> struct PvL { static hipError_t run(const Problem& p) { return launch_fwd_t<TR, D, kModePV>(p); } };
template <class TR, int D> struct FlashL {
  static hipError_t run(const Problem& p) {
    return p.ml ? launch_fwd_t<TR, D, kModeFlashML>(p) : launch_fwd_t<TR, D, kModeFlash>(p);
  }
};

}  // namespace

hipError_t launch_mfma_stats(const Problem& p) { return by_type<StatsL>(p); }
hipError_t launch_mfma_pv(const Problem& p) { return by_type<PvL>(p); }
hipError_t launch_mfma_flash(const Problem& p) { return by_type<FlashL>(p); }

}  // namespace attn
