// Matrix-core attention kernels for gfx950 (CDNA4): fp16 / bf16 operands,
// fp32 accumulation and fp32 softmax state.
//
// Method: "Speed Is All You Need: On-Device Acceleration of Large Diffusion
// Models via GPU-Aware Optimizations" (Chen et al.), news write-up, section on
// improving attention efficiency.  Two forms of O = softmax(scale Q K^T) V:
//   * partially fused softmax: fwd_kernel<.., kModeStats> reduces every row
//     of A = scale Q K^T to (m, l) -- the N x 2 tensor -- with the row's keys
//     cut into blocks that are reduced separately and merged in the same
//     launch; fwd_kernel<.., kModePV> then applies the softmax inside the
//     product with V.  A is recomputed from Q and K on chip, never stored.
//   * FlashAttention: fwd_kernel<.., kModeFlash*> walks the key blocks once
//     with a running max and running sum (exact online softmax).
// Exponentials are exp2 with scale * log2(e) folded in; (m, l) are reported
// in natural units.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>

#include "attn_internal.h"
#include "mfma_common.h"

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// Forward kernel: FlashAttention (online softmax), or either pass of the
// partially fused softmax.
//
// One workgroup = QG query groups of 32 queries x KH key splits (QG = 8, a
// 1024-thread workgroup per CU, at d = 40; 4 at d = 80; 2 at d = 160; halved
// when the problem has fewer workgroups than CUs; KH = 2, or 4 for those
// small d = 80 problems); the KH waves of a query group walk interleaved key
// blocks (the key range is cut into blocks as in the block-split reduction;
// 64-key blocks at d = 40 and for the single pass at d = 80 with two splits,
// 32 otherwise) and merge their partial (m, l, O) through LDS at the end.
// K and V blocks go through a ring of LDS slots per key split, filled
// cooperatively by that split's waves; more query groups per workgroup means
// fewer K/V copies per query from L2 into LDS.
//
//   * S^T = K Q^T on 32x32x16 MFMAs: a 32-key x 32-query tile per block, the
//     head dim in K=16 steps.  Lane l owns query l % 32 and 16 of the 32 keys;
//     lanes l and l ^ 32 share a query.
//   * one fp32 FMA per score forms x = c s - m (c = scale * log2(e), m the
//     reference max in exp2 units), and P = exp2(x).
//   * P is rounded to 16 bits, and one v_permlane16_swap per pair of packed
//     registers turns the 32x32 result layout into the B operands of two
//     16x16x32 MFMAs (queries 0-15 and 16-31) for O^T += V^T P^T.  V^T comes
//     from the [key][dim] LDS tile through ds_read_b64_tr_b16, in the key
//     order the swap produces.
//   * d = 40 pads the PV product to 48 rows; LDS column 40 of V holds 1.0 so
//     row 40 of O^T is the row sum l of the same rounded P.
// ---------------------------------------------------------------------------
// LDS row of key k of a V block (an involution): keys 16-19 and 20-23 (and
// their copies in every 32-key tile) trade places, so that the 8 rows one
// ds_read_b64_tr_b16 takes per half wave fall in distinct LDS banks.
__device__ __forceinline__ int vrow(int k) { return k ^ (((k >> 4) & 1) << 2); }

constexpr int kQ = 32;              // queries per wave

template <int D, int MODE, bool kHalfQ = false>
struct Shape {
  static constexpr int KS = (D + 15) / 16;      // K=16 steps of Q K^T
  static constexpr int MT = (D + 15) / 16;      // 16-row tiles of O^T
  static constexpr bool kOnes = (D % 16) != 0;  // LDS column D of V holds 1.0 -> O^T row D = l
  // LDS row pitches (16-bit elements), chosen with bank-conflict counters:
  // K rows are read 32 consecutive rows at a time by ds_read_b128 (pitch of
  // 20 or 28 words mod 64 reads in one pass); V rows by ds_read_b64_tr_b16 as
  // 4 rows x 32 bytes per 16 lanes (pitch of 24 or 40 words mod 64, with the
  // vrow permutation); d = 40 needs padding columns 40..47 in both.
  static constexpr int PK = D == 40 ? 56 : D + 8;
  static constexpr int PV = D == 40 ? 48 : (D == 80 ? 80 : D + 16);
  // keys per block: 64 at d = 40, and at d = 80 for the single pass (measured
  // 7-13 % faster there; the two-pass form stays at 32, where 64 was slower at
  // N >= 4096); 32 otherwise
  static constexpr bool kFlashLike = MODE == kModeFlash || MODE == kModeFlashML;
  // key splits per query group: 2, or 4 for the small d = 80 problems that
  // take the halved shape (twice the waves; 32-key blocks keep the four
  // rings within LDS)
  static constexpr int KH = (kHalfQ && D == 80) ? 4 : 2;
  static constexpr int BN = (D == 40 || (D == 80 && kFlashLike && KH == 2)) ? 64 : 32;
  // query groups per workgroup: d = 160 takes 2 (half the workgroup, twice
  // the workgroups for the small sequences of the UNet's deep levels);
  // kHalfQ halves it again for problems with fewer workgroups than CUs
  static constexpr int QG0 = D == 40 ? 8 : (D == 160 ? 2 : 4);
  static constexpr int QG = kHalfQ && QG0 > 1 ? QG0 / 2 : QG0;
  static constexpr int W = KH * QG;              // waves per workgroup
  static constexpr int T = 64 * W;               // threads per workgroup
  static constexpr int HT = 64 * QG;             // threads per key split
  static constexpr int QWG = QG * kQ;            // queries per workgroup
  static constexpr int NT = BN / 32;             // 32-key score tiles per block
  static constexpr int NBUF = D >= 160 ? 2 : 3;  // ring slots per key split
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int SLOT = BN * (PK + PV);    // 16-bit elements per slot (K then V)
  static_assert(D % 8 == 0 && D >= 16, "head dim must be a multiple of 8");
};

template <class TR, int D, int MODE, bool kHalfQ>
__global__ __launch_bounds__((Shape<D, MODE, kHalfQ>::T)) void fwd_kernel(const uint16_t* __restrict__ q,
                                                 const uint16_t* __restrict__ k,
                                                 const uint16_t* __restrict__ v,
                                                 uint16_t* __restrict__ out,
                                                 float* __restrict__ ml, const float* __restrict__ a,
                                                 const Layout lay, int Nq, int Nk, int qtiles, int nwg,
                                                 float scale) {
  using S = Shape<D, MODE, kHalfQ>;
  constexpr int KS = S::KS, MT = S::MT, PK = S::PK, PV = S::PV, NBUF = S::NBUF;
  constexpr int BN = S::BN, NT = S::NT, kQG = S::QG, kHT = S::HT, kQWG = S::QWG, KH = S::KH;
  constexpr bool kStats = MODE == kModeStats;
  constexpr bool kFromA = MODE == kModePVScores;             // logits read from A (float32)
  constexpr bool kPVLike = MODE == kModePV || kFromA;        // (m, l) given, O only
  constexpr bool kReportML = MODE == kModeFlashML || kStats;
  // where l comes from: the matrix cores (V's ones column in the flash forms)
  // or fp32 sums of the unrounded P on the vector ALU (the stats form: its
  // P feeds no product, so it is never packed; measured 8 % faster than a
  // sum of the packed P on the matrix cores)
  constexpr bool kValuSum = !kPVLike && (kStats || !S::kOnes || (kReportML && !TR::kRoundedSumOk));
  constexpr int MO = kStats ? 1 : MT;  // 16-row tiles of the accumulator (none used in the stats form)
  // floats per lane handed from one key split to the first in the merge: O
  // (not in the stats form), then 4 per query tile
  constexpr int XO = kStats ? 0 : 2 * MT * 4, NEX = XO + 8;
  // LDS slot: the K block, then the V block (none in the stats form)
  constexpr int SLOT = kStats ? BN * PK : S::SLOT;
  // LDS: a ring per key split; after the walk, an exchange area per split
  // but the first (floats, counted here in 16-bit elements)
  constexpr int RING = KH * NBUF * SLOT, XCH = NEX * 64 * kQG * (KH - 1) * 2;
  constexpr int SMEM = RING > XCH ? RING : XCH;
  // fp16 flash without (m, l) out: the rescale test runs on the packed P
  constexpr bool kLazyMax = TR::kPackedMax && MODE == kModeFlash;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int qg = wave % kQG, split = wave / kQG, htid = tid % kHT;
  const int l32 = lane & 31, hi = lane >> 5;  // 32x32 layout: query l32, key subgroup hi
  const int G = lane >> 4, li = lane & 15;    // 16x16 layout
  // exp2 units: the stored A already carries the scale
  const float c = kFromA ? kLog2e : scale * kLog2e;

  const int tile = xcd_tile(nwg);
  const int head = tile / qtiles;
  const int qbase = (tile - head * qtiles) * kQWG + qg * kQ;
  const uint16_t* qh = q + head_offset(lay.q, lay.H, head);
  const uint16_t* kh = k + head_offset(lay.k, lay.H, head);
  const uint16_t* vh = kStats ? nullptr : v + head_offset(lay.v, lay.H, head);  // the stats form reads no V
  const int qrs = lay.q.row, krs_ = lay.k.row, vrs_ = lay.v.row;  // row strides (elements)
  uint16_t* const ring = smem + split * NBUF * SLOT;

  if constexpr (S::kOnes) {
    // padding columns of every slot of this split: zero, except V column D =
    // 1.0 (the row-sum dim)
    for (int e = htid; e < NBUF * BN * (PK - D); e += kHT) {
      const int r = e / (PK - D), col = e - r * (PK - D);
      ring[(r / BN) * SLOT + (r % BN) * PK + D + col] = 0;
    }
    for (int e = htid; !kStats && e < NBUF * BN * (PV - D); e += kHT) {
      const int r = e / (PV - D), col = e - r * (PV - D);
      ring[(r / BN) * SLOT + BN * PK + (r % BN) * PV + D + col] = col == 0 ? TR::kOne : (uint16_t)0;
    }
  }

  // Reference max in exp2 units, per query (lane l32): the value subtracted
  // (in fp32) from every score.  The online form starts from 0 and always
  // re-bases on its first block.
  float mref = 0.f;
  if constexpr (kPVLike) {
    const int row = qbase + l32;
    mref = row < Nq ? ml[((size_t)head * Nq + row) * 2] * kLog2e : 0.f;  // stored in natural units
  }
  // Q operand (B of the 32x32x16 MFMA): query l32, dims [16 ks + 8 hi, +8),
  // zero past d.  The scale stays out of the 16-bit operand: rounding c * q
  // to 16 bits would move a score by up to 2^-11 of its own size, which is
  // visible in P once scores reach tens.
  s8v qf[KS];
  if constexpr (kFromA) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = (s8v){0, 0, 0, 0, 0, 0, 0, 0};  // Q is not read
  } else {
    const int row = qbase + l32;
    const bool ok = row < Nq;
    const uint16_t* qp = qh + (size_t)(ok ? row : 0) * qrs;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 16 + hi * 8;
      const uint4 x = *(const uint4*)(qp + (d0 < D ? d0 : D - 8));
      qf[ks] = (ok && d0 < D) ? __builtin_bit_cast(s8v, x) : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // state: O in the 16x16 layout; the max in exp2 units in the 32x32 layout
  f4v o[2][MO];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int mt = 0; mt < MO; ++mt) o[qt][mt] = (f4v){0.f, 0.f, 0.f, 0.f};
  float mtrue = -INFINITY, lsum = 0.f;

  const int nblk = (Nk + BN - 1) / BN;
  const int niter = (nblk + KH - 1) / KH;
  // Staging of this split's block for iteration `it` (key block KH it +
  // split).  One job = one 16-byte chunk per lane, one buffer load and one
  // ds_write_b128 per wave; the split's waves take jobs qg, qg + QG, ...  K
  // chunks go column by column (lane -> key row), V chunks in LDS order over
  // the permuted key rows; both orders write LDS without bank conflicts.  The
  // buffer resource starts at the block's first key and ends at key Nk, so
  // the block address is scalar work and rows past Nk come back as zeros.
  constexpr int VCH = PV / 8;                                 // chunks per V row (incl. padding)
  // (reading A, the K blocks are not needed)
  constexpr int KJOBS = kFromA ? 0 : BN * S::CPR / 64, NJOB = KJOBS + (kStats ? 0 : (BN * VCH + 63) / 64);
  constexpr int JPW = (NJOB + kQG - 1) / kQG;                 // jobs per wave
  static_assert(BN * S::CPR % 64 == 0, "K staging covers whole waves");
  // A rows of this head (float32 [Nq][Nk]): lane l32 reads row qbase + l32
  // (rows past Nq are past the resource and read as zero)
  const __amdgpu_buffer_rsrc_t ars =
      make_rsrc(kFromA ? (const void*)(a + (size_t)head * Nq * Nk) : (const void*)kh, kFromA ? Nq * Nk * 4 : 0);
  const int arow = (qbase + l32) * Nk;
  const int splitu = __builtin_amdgcn_readfirstlane(split);
  const int qgu = __builtin_amdgcn_readfirstlane(qg);
  int goff[JPW], soff[JPW];  // byte offset in the block (< 0: no chunk), element offset in the slot
#pragma unroll
  for (int r = 0; r < JPW; ++r) {
    const int j = qgu + kQG * r;
    goff[r] = -1;
    soff[r] = 0;
    if (j < KJOBS) {
      const int qi = 64 * j + lane, col = qi / BN, row = qi - col * BN;
      goff[r] = (row * krs_ + col * 8) * 2;
      soff[r] = row * PK + col * 8;
    } else if (j < NJOB) {
      const int qi = 64 * (j - KJOBS) + lane, row = qi / VCH, col = qi - row * VCH;
      if (row < BN && col < S::CPR) {
        goff[r] = (vrow(row) * vrs_ + col * 8) * 2;
        soff[r] = BN * PK + row * PV + col * 8;
      }
    }
  }
  uint4 stg[JPW];
  auto gload = [&](int it) {
    const int key0 = (KH * it + splitu) * BN;
    // the resources end after the last key's d elements
    // up to 2^32 - 2 bytes (a head holds fewer than 2^31 elements): unsigned
    const unsigned kbytes = Nk > key0 ? ((unsigned)(Nk - key0 - 1) * (unsigned)krs_ + D) * 2u : 0u;
    const unsigned vbytes = Nk > key0 ? ((unsigned)(Nk - key0 - 1) * (unsigned)vrs_ + D) * 2u : 0u;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kh + (size_t)key0 * krs_, kbytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc((kStats ? kh : vh) + (size_t)key0 * vrs_, kStats ? 0 : vbytes);
#pragma unroll
    for (int r = 0; r < JPW; ++r) {
      const int j = qgu + kQG * r;
      if (j < NJOB) stg[r] = load16(j < KJOBS ? krs : vrs, goff[r] < 0 ? 0x7FFFFFF0 : goff[r]);
    }
  };
  auto swrite = [&](int slot) {
    uint16_t* sl = ring + slot * SLOT;
#pragma unroll
    for (int r = 0; r < JPW; ++r)
      if (qgu + kQG * r < NJOB && goff[r] >= 0) *(uint4*)(sl + soff[r]) = stg[r];
  };

#pragma unroll
  for (int d = 0; d + 1 < NBUF; ++d) {
    if (d < niter) {
      gload(d);
      swrite(d);
    }
  }
  // Everything loaded so far (Q, first blocks) is complete here; saying so
  // keeps the compiler from waiting on the in-flight prefetch inside the loop.
  wait_vmem_all();
  __syncthreads();
  if (NBUF - 1 < niter) gload(NBUF - 1);

  // key order after the row swap: lane group G holds keys vbase + {0..3} and
  // vbase + 8 + {0..3}, at LDS rows vrow(vbase) + {0..3}, + 8 + {0..3}
  const int vbase = vrow((G & 1) * 16 + (G >> 1) * 4);

  // Online softmax.  The reference max moves only when a block's scores
  // exceed it by more than 8 (exp2 units), so P = exp2(x) <= 256 stays exact
  // in 16-bit P and in the fp32 sums; O / l does not depend on the reference.
  // move the reference to the running max, rescale O and l, and shift the
  // block's scores
  auto rebase = [&](f16v (&x)[NT], float bm) {
    mtrue = __builtin_fmaxf(mtrue, bm + mref);
    const float delta = mtrue - mref;
    const float alpha = __builtin_amdgcn_exp2f(-delta);
    mref = mtrue;
    lsum *= alpha;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[t][i] -= delta;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float ao = __shfl(alpha, qt * 16 + li);
#pragma unroll
      for (int mt = 0; mt < MO; ++mt) o[qt][mt] *= ao;
    }
  };
  auto block_max = [&](const f16v (&x)[NT]) {
    float bm = x[0][0];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) bm = __builtin_fmaxf(bm, x[t][i]);
    return pair_max32(bm);  // both lanes of a query
  };
  // P = exp2(x) rounded to 16 bits, re-laid out for the PV product:
  // pa[t]: queries 0-15, pb[t]: queries 16-31; returns the fp32 sum of P
  uint32_t pa[NT][4], pb[NT][4];
  auto expand = [&](const f16v (&x)[NT]) {
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(x[t][i]);
      if constexpr (kValuSum) {
#pragma unroll
        for (int i = 0; i < 16; ++i) ls += p[i];
      }
#pragma unroll
      for (int d = 0; d < (kStats ? 0 : 4); ++d) {
        pa[t][d] = TR::pack2(p[2 * d], p[2 * d + 1]);
        pb[t][d] = TR::pack2(p[8 + 2 * d], p[8 + 2 * d + 1]);
        swap16(pa[t][d], pb[t][d]);
      }
    }
    return ls;
  };

  for (int it = 0; it < niter; ++it) {
    const int kb = KH * it + splitu;  // wave-uniform
    if (kb < nblk) {
      const uint16_t* Ks = ring + (it % NBUF) * SLOT;
      const uint16_t* Vs = Ks + BN * PK;
      // ---- scores in exp2 units relative to mref, NT tiles of 32 keys x 32 queries
      f16v x[NT];
      // raised wave priority while issuing matrix work, so that a wave with
      // MFMAs ready goes first and the others' vector work fills the gaps
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        x[t] = (f16v){};
        if constexpr (kFromA) {
          // the same 32x32 layout, from memory: keys (i/4)*8 + hi*4 + (i%4) of the tile
          const int k0 = kb * BN + t * 32 + hi * 4;
          if ((Nk & 3) == 0) {  // rows start 16-byte aligned: 4 keys per load
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f4v y = __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(ars, (arow + k0 + g * 8) * 4, 0, 0));
#pragma unroll
              for (int j = 0; j < 4; ++j) x[t][4 * g + j] = y[j];
            }
          } else {
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                x[t][4 * g + j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ars, (arow + k0 + g * 8 + j) * 4, 0, 0));
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int d0 = ks * 16 + hi * 8;
            // past d the LDS padding is zero (and so is Q)
            const s8v a = *(const s8v*)(Ks + (t * 32 + l32) * PK + d0);
            x[t] = TR::mma32(a, qf[ks], x[t]);
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) x[t][i] = __builtin_fmaf(x[t][i], c, -mref);
      }
      __builtin_amdgcn_s_setprio(0);
      if (kb * BN + BN > Nk) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb * BN + t * 32 + (i / 4) * 8 + hi * 4 + (i % 4) >= Nk) x[t][i] = -INFINITY;
      }
      float ls;
      if constexpr (kLazyMax) {
        // exponentials first: the 16-bit P themselves tell whether a score
        // passed mref + 8 (P > 256); only then is the block max taken and P
        // formed again against the new reference
        ls = expand(x);
        uint32_t mw = pa[0][0];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int d = 0; d < 4; ++d) mw = pmax(pmax(mw, pa[t][d]), pb[t][d]);
        if (__any(pmax_halves(mw) > 256.f) || it == 0) {
          rebase(x, block_max(x));
          ls = expand(x);
        }
      } else {
        if constexpr (!kPVLike) {
          const float bm = block_max(x);
          if (__any(bm > 8.f) || it == 0) rebase(x, bm);
          else mtrue = __builtin_fmaxf(mtrue, bm + mref);
        }
        ls = expand(x);
      }
      if constexpr (kValuSum) lsum += ls;
      // ---- O^T += V^T P^T; lane (G, li) supplies V^T[dim 16 mt + li][its 8 keys]
      // (the stats form has no product: its P were summed above)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < (kStats ? 0 : NT); ++t) {
        const s8v P0 = __builtin_bit_cast(s8v, (uint4){pa[t][0], pa[t][1], pa[t][2], pa[t][3]});
        const s8v P1 = __builtin_bit_cast(s8v, (uint4){pb[t][0], pb[t][1], pb[t][2], pb[t][3]});
        const uint16_t* Vt = Vs + t * 32 * PV;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint16_t* va = Vt + (vbase + (li >> 2)) * PV + mt * 16 + 4 * (li & 3);
          const s4v v0 = lds_read_tr16(va);
          const s4v v1 = lds_read_tr16(va + 8 * PV);
          const s8v vop = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          o[0][mt] = TR::mma16(vop, P0, o[0][mt]);
          o[1][mt] = TR::mma16(vop, P1, o[1][mt]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (it + NBUF - 1 < niter) swrite((it + NBUF - 1) % NBUF);
    __syncthreads();
    if (it + NBUF < niter) gload(it + NBUF);
  }

  // ---- per-query state in the 16x16 layout: lane (G, li) <- query qt*16 + li
  if (nblk <= split) mref = -INFINITY;  // this split saw no key: it must not weigh in the merge
  float mo[2], mto[2], lo[2], lro[2];
  const float lfull = kValuSum ? pair_sum32(lsum) : 0.f;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    mo[qt] = __shfl(mref, qt * 16 + li);
    mto[qt] = __shfl(mtrue, qt * 16 + li);
    if constexpr (kPVLike) {
      lo[qt] = 0.f;
      lro[qt] = 0.f;
    } else {
      if constexpr (S::kOnes && !kStats) {
        constexpr int GL = (D % 16) / 4, IL = D % 4;
        lo[qt] = __shfl(o[qt][MT - 1][IL], GL * 16 + li);
      } else {
        lo[qt] = __shfl(lfull, qt * 16 + li);
      }
      lro[qt] = kValuSum ? __shfl(lfull, qt * 16 + li) : lo[qt];
    }
  }

  // ---- merge the key splits: splits 1 .. KH-1 hand their state to split 0
  // through LDS, which folds them in, in that order
  float* const ex0 = (float*)smem + lane;
  auto exch = [&](int sp) { return ex0 + ((sp - 1) * kQG + qg) * NEX * 64; };
  if (split > 0) {
    float* ex = exch(split);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int mt = 0; mt < (kStats ? 0 : MT); ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) ex[((qt * MT + mt) * 4 + i) * 64] = o[qt][mt][i];
      ex[(XO + qt * 4 + 0) * 64] = mo[qt];
      ex[(XO + qt * 4 + 1) * 64] = mto[qt];
      ex[(XO + qt * 4 + 2) * 64] = lo[qt];
      ex[(XO + qt * 4 + 3) * 64] = lro[qt];
    }
  }
  __syncthreads();
  if (split > 0) return;
#pragma unroll
  for (int sp = 1; sp < KH; ++sp) {
    const float* ex = exch(sp);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float mB = ex[(XO + qt * 4 + 0) * 64];
      const float mtB = ex[(XO + qt * 4 + 1) * 64];
      const float lB = ex[(XO + qt * 4 + 2) * 64];
      const float lrB = ex[(XO + qt * 4 + 3) * 64];
      // the sums below are written as explicit FMAs: left to the compiler,
      // the contraction may differ between the workgroup shapes and with it
      // the last bit of O
      float fA = 1.f, fB = 1.f, M = mo[qt];
      if constexpr (!kPVLike) {
        // a split that saw no key holds (-inf, 0, 0) and contributes nothing
        M = __builtin_fmaxf(mo[qt], mB);
        fA = __builtin_amdgcn_exp2f(mo[qt] - M);
        fB = __builtin_amdgcn_exp2f(mB - M);
      }
#pragma unroll
      for (int mt = 0; mt < (kStats ? 0 : MT); ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[qt][mt][i] = __builtin_fmaf(o[qt][mt][i], fA, ex[((qt * MT + mt) * 4 + i) * 64] * fB);
      lo[qt] = __builtin_fmaf(lo[qt], fA, lB * fB);
      lro[qt] = __builtin_fmaf(lro[qt], fA, lrB * fB);
      mto[qt] = __builtin_fmaxf(mto[qt], mtB);
      mo[qt] = M;
    }
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float M = mo[qt], l = lo[qt], lr = lro[qt], mt_all = mto[qt];
    const int row = qbase + qt * 16 + li;
    float inv = 0.f;
    if (row < Nq) {
      if constexpr (kPVLike) {
        // P was formed against mref = the given m (M here); the given l is
        // relative to it
        const float2 st = *(const float2*)(ml + ((size_t)head * Nq + row) * 2);
        inv = __builtin_amdgcn_exp2f(__builtin_fmaf(-st.x, kLog2e, M)) / st.y;
      } else {
        inv = 1.f / l;
      }
    }
    if (row < Nq) {
      uint16_t* op = out + head_offset(lay.o, lay.H, head) + (size_t)row * lay.o.row;
#pragma unroll
      for (int mt = 0; mt < (kStats ? 0 : MT); ++mt) {
        const int dim = mt * 16 + G * 4;
        if (dim < D) {
          uint2 w;
          w.x = TR::pack2(o[qt][mt][0] * inv, o[qt][mt][1] * inv);
          w.y = TR::pack2(o[qt][mt][2] * inv, o[qt][mt][3] * inv);
          *(uint2*)(op + dim) = w;
        }
      }
      if constexpr (kReportML) {
        if (G == 0) {
          // l was accumulated against the reference M; report it against the true max
          const float lt = lr * __builtin_amdgcn_exp2f(M - mt_all);
          *(float2*)(ml + ((size_t)head * Nq + row) * 2) = make_float2(mt_all / kLog2e, lt);
        }
      }
    }
  }
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev] = n;  // the same value from every thread: a benign race
  }
  return counts[dev];
}

template <class TR, int D, int MODE, bool kHalfQ>
hipError_t launch_fwd_q(const Problem& p, int qtiles, long long nwg) {
  hipLaunchKernelGGL((fwd_kernel<TR, D, MODE, kHalfQ>), dim3((unsigned)nwg), dim3((Shape<D, MODE, kHalfQ>::T)), 0,
                     p.stream, (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v, (uint16_t*)p.out,
                     p.ml, p.a, p.lay, p.Nq, p.Nk, qtiles, (int)nwg, p.scale);
  return hipGetLastError();
}

// Workgroups of the default shape when they fill the chip; otherwise half
// the query groups per workgroup and twice the workgroups (every wave does
// the same work either way, so the results are identical), and at d = 80
// also four key splits of 32-key blocks instead of two (twice the waves; the
// key blocking differs, so the results agree to rounding, not bit for bit).
template <class TR, int D, int MODE>
hipError_t launch_fwd_t(const Problem& p) {
  using S = Shape<D, MODE, false>;
  using H = Shape<D, MODE, true>;
  const int qtiles = (p.Nq + S::QWG - 1) / S::QWG;
  const long long nwg = (long long)p.BH * qtiles;
  if (H::QG < S::QG && nwg < cu_count()) {
    const int qt2 = (p.Nq + H::QWG - 1) / H::QWG;
    return launch_fwd_q<TR, D, MODE, true>(p, qt2, (long long)p.BH * qt2);
  }
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  return launch_fwd_q<TR, D, MODE, false>(p, qtiles, nwg);
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

// Whether a head-dimension-40 problem takes the kernel of attn_fa40.hip or
// this file's.  Measured on MI355X (both kernels on one box, B=2, H=8,
// per-launch medians, graph-replayed launches alike): the attn_fa40.hip kernel
// is faster from 1536 keys on, by 3-11 % at Nq = 4096 (1536-16384 keys) and
// 2-11 % at Nq = 16384 (1536-16384 keys, Q, K ~ N(0, 1.5^2)), level at 1024
// keys and slower at 512; so it takes every problem with more than 1024 keys.
// ATTN_FA40=0 turns it off, ATTN_FA40=1 forces it wherever d = 40 (for
// comparisons).
bool use_fa40(const Problem& p, int cus) {
  const char* e = std::getenv("ATTN_FA40");  // (read per launch: tests switch it)
  if (e && (e[0] == '0' || e[0] == '1')) return e[0] == '1';
  (void)cus;
  return p.Nk > 1024;
}

// Whether a single pass takes the short-key-range kernel of attn_short.hip:
// every key range it supports (with at most 65535 heads and batches: its
// grid's y and z dimensions).  ATTN_SHORT=0 turns it off (for comparisons;
// =s / =w select its shared / per-wave form where the shape allows).
bool use_short(const Problem& p) {
  if (p.Nk > short_max_keys(p.d) || p.lay.H > 65535 || p.BH / p.lay.H > 65535) return false;
  const char* e = std::getenv("ATTN_SHORT");  // (read per launch: tests switch it)
  return !(e && e[0] == '0');
}

template <class TR, int D> struct StatsL { static hipError_t run(const Problem& p) { return launch_fwd_t<TR, D, kModeStats>(p); } };
template <class TR, int D> struct PvL {
  static hipError_t run(const Problem& p) {
    if (D == 40 && use_fa40(p, cu_count())) return launch_fa40_pv(p, cu_count());
    return launch_fwd_t<TR, D, kModePV>(p);
  }
};
template <class TR, int D> struct PvAL { static hipError_t run(const Problem& p) { return launch_fwd_t<TR, D, kModePVScores>(p); } };
template <class TR, int D> struct FlashL {
  static hipError_t run(const Problem& p) {
    if (use_short(p)) return launch_short_flash(p, cu_count());
    if (D == 40 && use_fa40(p, cu_count())) return launch_fa40_flash(p, cu_count());
    return p.ml ? launch_fwd_t<TR, D, kModeFlashML>(p) : launch_fwd_t<TR, D, kModeFlash>(p);
  }
};

}  // namespace

hipError_t launch_mfma_stats(const Problem& p) { return by_type<StatsL>(p); }
hipError_t launch_mfma_pv(const Problem& p) { return by_type<PvL>(p); }
hipError_t launch_mfma_pv_scores(const Problem& p) { return by_type<PvAL>(p); }
hipError_t launch_mfma_flash(const Problem& p) { return by_type<FlashL>(p); }

}  // namespace attn
