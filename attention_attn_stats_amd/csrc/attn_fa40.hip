// Software-pipelined matrix-core attention at head dimension 40 (the SD UNet's
// top level), fp16 / bf16 operands, fp32 accumulation and softmax state.
//
// Method: "Speed Is All You Need: On-Device Acceleration of Large Diffusion
// Models via GPU-Aware Optimizations" (Chen et al.), news write-up, section on
// improving attention efficiency: the single-pass FlashAttention form (keys
// walked in tiles with a running softmax state, exact) and the second pass of
// the partially fused softmax (the softmax applied inside the product with V,
// from the row statistics of the first pass).
//
// Design for gfx950 (one wave = 32 queries; 16 waves per CU):
//  * S^T = K Q^T on v_mfma_f32_32x32x16 (a 32-key tile, the head dim in three
//    K=16 steps).  O^T += V^T P^T in two parts: dims 0-31 as one 32-row tile
//    on v_mfma_f32_32x32x16, whose B-operand layout is the 32x32 result
//    layout of S^T once its keys are renumbered (P goes from the exponentials
//    straight into the product); dims 32-47 (dims 32-39, the row sum, zeros)
//    as two 16x16x32 products, one per 16 queries, on P re-laid out by four
//    v_permlane16_swap per tile (a 32-row tile there would be 23/32 padding).
//    V^T comes from LDS in the matching key orders through ds_read_b64_tr_b16.
//  * Row 40 of V^T is 1.0 for every key, so row 40 of O^T is the row sum l
//    of the same rounded P the numerator used.
//  * Each wave runs a software pipeline over 32-key tiles: while the vector
//    ALU forms P of tile t (one FMA, one exp2, half a pack per score; no FMA
//    in the fp16 O-only form), the matrix cores compute the scores of tile
//    t+1 and accumulate P of tile t-1 into O, so one wave alone keeps both
//    units fed.
//  * K and V blocks (64 keys) reach LDS by direct buffer-to-LDS loads into a
//    four-slot ring per key split, issued two blocks ahead and waited for just
//    before the one barrier per block; no registers hold staged data.
//  * The single pass keeps one reference max per query: the exact max of the
//    first tile (in fp16, 4 exp2 units above it).  Scores beyond the reference
//    by up to 16 keep P finite in fp16; a row whose sum comes out non-finite
//    or above 2^50 is recomputed by
//    the whole workgroup with a reference that follows the running max tile
//    by tile (exact online softmax), so the fast path needs no per-tile test.
//  * fp16, O only: after the first tile Q is scaled by scale * log2(e) and
//    rounded to fp16, and dim 41 of Q holds -reference against a K dim 41 of
//    1.0, so the score product itself yields the exp2 argument.  The scaled
//    Q's rounding (2^-11 of each product term) is the form's one extra error;
//    a reference beyond +-64, or a scaled element beyond fp16's range, sends
//    the workgroup to the exact pass.
//  * Keys past Nk: their K rows and V rows read as zero (buffer range check)
//    and a mask column (K dim 40 = 1 for them, 0 otherwise, against a query
//    dim 40 of -2^15) drives their scores to -2^15 * scale, so exp2 gives 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "mfma_common.h"

namespace attn {
namespace {

namespace fa40 {

constexpr int D = 40;
constexpr int BN = 64;         // keys per block (two 32-key tiles)
constexpr int NBUF = 4;        // ring slots per key split
constexpr int KH = 2;          // key splits per query group
// K block: 64 rows of 112 bytes (7 chunks of 16 B: dims 0-39, the mask
// chunk (dim 40 the mask, dim 41 the 1.0 of the folded reference), one
// unused); the 28-word pitch reads 16 consecutive rows by ds_read_b128
// without bank conflicts.
constexpr int KPITCH = 112;
constexpr int KCH = 7;
constexpr int KBYTES = BN * KPITCH;               // 7168
// V block: groups of 4 keys, each 6 chunks x 4 keys (chunk c of key 4j+t at
// chunk position 24j + 4c + t); chunk 5 holds (1, 0, ..., 0): the row-sum
// dim 40 and zero dims 41-47.  A transposed read of 4 keys x 32 dims touches
// 16 distinct 16-byte bank groups.
constexpr int VGRP = 24;
constexpr int VBYTES = (BN / 4) * VGRP * 16;      // 6144
constexpr int SLOT = KBYTES + VBYTES;             // 13312
constexpr int RING = NBUF * SLOT;                 // 53248 per key split
constexpr int KJOBS = KBYTES / 1024;              // 7 direct loads of 64 x 16 B
constexpr int VJOBS = VBYTES / 1024;              // 6
constexpr int NJOBS = KJOBS + VJOBS;              // 13
constexpr int DUMMY = 2 * RING;                   // 1 KB that out-of-range padding loads fill with zeros
// a row whose fast-path sum is not below this is recomputed (P up to
// 65504 per key in fp16; bf16 P never overflows, the bound keeps O finite)
constexpr float kSumLimit = 1125899906842624.f;   // 2^50
// fp16 fast path: the reference max lies this far (exp2 units) above the
// first tile's max.  A later score more than 16 above the reference makes P
// leave the fp16 range and the whole workgroup redo its rows; with logits of
// standard deviation ~2.25 (Q, K ~ N(0, 1.5^2) at d = 40) a 16-unit gap above
// the first 32 keys' max occurs in a few rows of a 4096 x 4096 launch, and one
// such row doubles its workgroup's time.  At 4 the gap needed is 20; the
// first tile's max key weighs 2^-4, a P stays in the fp16 normal range down to
// 2^-14 (keys 10 below that max), and each one rounded in the denormal range
// errs by at most 2^-25, i.e. 2^-21 of the row sum.
constexpr float kHeadroom = 4.f;

template <int QG>
struct Cfg {
  static constexpr int W = KH * QG;          // waves per workgroup
  static constexpr int T = 64 * W;
  static constexpr int HT = 64 * QG;         // threads per key split
  static constexpr int QWG = 32 * QG;        // queries per workgroup
  // direct loads per wave and block: the same count for every wave (waves
  // past the 13 jobs issue out-of-range loads into a padding area), so that
  // the waits before each barrier are compile-time counts
  static constexpr int MAXJ = (NJOBS + QG - 1) / QG;
  static constexpr int XN = 24;              // floats per lane handed over in the split merge
  static_assert((KH - 1) * QG * XN * 64 * 4 <= KH * RING, "merge area within the ring");
  static constexpr int SMEM = KH * RING + 1024;
};

typedef __attribute__((address_space(3))) uint8_t lds8;

__device__ __forceinline__ s8v lds_read_b128(const lds8* p) {
  return *(const __attribute__((address_space(3))) s8v*)p;
}
// 16-byte LDS store of four words
__device__ __forceinline__ void lds_store16(lds8* p, uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  typedef uint32_t __attribute__((ext_vector_type(4))) u4v;
  *(__attribute__((address_space(3))) u4v*)p = (u4v){x0, x1, x2, x3};
}
// 16 bytes per lane from a buffer resource straight into LDS at dst + 16 lane
// (dst wave-uniform); out-of-range lanes write zeros
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, lds8* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}
// C += A B on v_mfma_f32_16x16x32 with the accumulator kept in its registers
// (destination = accumulator input): the LDS reads of the next tile may then
// reuse no register the product still reads.  The two wait states cover a
// vector-ALU write of A or B just before (the exchanged P).
template <class TR>
__device__ __forceinline__ void mma16_acc(s8v a, s8v b, f4v& c) {
  if constexpr (TR::kPackedMax)
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  else
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ s4v lds_tr(const lds8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s4v __attribute__((address_space(3)))*)p);
}
// s_waitcnt vmcnt(n), n < 16 (expcnt, lgkmcnt at their no-wait maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
// lgkmcnt(0): every LDS access of this wave complete
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier that orders LDS and direct-load traffic only through the
// explicit waits placed before it (the library's own __syncthreads would also
// wait for every outstanding direct load, which defeats loading ahead); the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The per-lane constants of a wave's direct loads: for its r-th job of a
// block, the byte offset of its 16-byte chunk within the block in global
// memory and whether the lane loads (the V block's ones chunks and the K
// rows' mask and spare chunks are not loaded).
template <int QG>
struct Dma {
  int voff[Cfg<QG>::MAXJ];
  bool act[Cfg<QG>::MAXJ];
};

// The row sum l of query l32 (row 40 of O^T in the 16x16 layout: register 0
// of lanes 32-47 of the queries-0-15 tile a or the queries-16-31 tile b).
__device__ __forceinline__ float row_sum(float a, float b, int l32) {
  const float la = __shfl(a, 32 + (l32 & 15)), lb = __shfl(b, 32 + (l32 & 15));
  return l32 < 16 ? la : lb;
}

// Q^T operand of the score product for query `row` (rows past Nq read as
// zero): lane half hi holds dims 16 ks + 8 hi .. + 7; dims 40-47 hold the
// mask weight -2^15 (dim 40) and zeros
template <class TR>
__device__ __forceinline__ void load_q_operand(s8v (&qf)[3], const uint16_t* qh, int qrow_stride, int row, int hi,
                                               int Nq) {
  const bool ok = row < Nq;
  const uint16_t* qp = qh + (size_t)(ok ? row : 0) * qrow_stride;
#pragma unroll
  for (int ks = 0; ks < 3; ++ks) {
    const int d0 = ks * 16 + hi * 8;
    if (d0 < D) {
      const uint4 x = *(const uint4*)(qp + d0);
      qf[ks] = ok ? __builtin_bit_cast(s8v, x) : (s8v){0, 0, 0, 0, 0, 0, 0, 0};
    } else {
      qf[ks] = (s8v){(short)TR::kMinus2p15, 0, 0, 0, 0, 0, 0, 0};
    }
  }
}

}  // namespace fa40

// ---------------------------------------------------------------------------
// fa40_kernel<TR, MODE, QG>: MODE = kModeFlash (O), kModeFlashML (O and
// (m, l)) or kModePV (O from given (m, l)).  Workgroup = QG query groups of
// 32 queries x 2 key splits; split s walks key blocks s, s + 2, ...; the
// splits merge (m, O) through LDS at the end.
// ---------------------------------------------------------------------------
template <class TR, int MODE, int QG>
__global__ __launch_bounds__((fa40::Cfg<QG>::T)) void fa40_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            uint16_t* __restrict__ out, float* __restrict__ ml,
                                                            const Layout lay, int Nq, int Nk, int qtiles, int nwg,
                                                            float scale) {
  using namespace fa40;
  using C = Cfg<QG>;
  constexpr bool kPV = MODE == kModePV;
  constexpr bool kML = MODE == kModeFlashML;
  // bf16-rounded P is too coarse for a reported l: sum the fp32 P as well
  constexpr bool kValuSum = kML && !TR::kRoundedSumOk;
  // fp16 O-only fast path: the scale and the reference max go into the score
  // product (Q scaled into exp2 units in fp16, -reference against a K dim of
  // 1.0), so that P is exp2 of the product's result with no vector FMA
  constexpr bool kFold = MODE == kModeFlash && TR::kPackedMax;
  __shared__ __attribute__((aligned(16))) uint8_t smem_[C::SMEM];
  __shared__ int redo_flag;
  // the LDS address of the array (a generic pointer into LDS keeps it in its low 32 bits)
  lds8* const smem = (lds8*)(uintptr_t)(uint32_t)(uintptr_t)smem_;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int qg = wave % QG, split = wave / QG;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qgu = __builtin_amdgcn_readfirstlane(qg);
  const int splitu = __builtin_amdgcn_readfirstlane(split);
  const float c = scale * kLog2e;  // exp2 units

  const int tile = xcd_tile(nwg);
  const int head = tile / qtiles;
  const int qbase = (tile - head * qtiles) * C::QWG + qg * 32;
  const uint16_t* qh = q + head_offset(lay.q, lay.H, head);
  const uint16_t* kh = k + head_offset(lay.k, lay.H, head);
  const uint16_t* vh = v + head_offset(lay.v, lay.H, head);
  const int krs = lay.k.row, vrs = lay.v.row;
  lds8* const ring = smem + splitu * RING;

  const int nblk = (Nk + BN - 1) / BN;
  const int nb = (nblk - splitu + KH - 1) / KH;     // blocks of this split
  const int niter = (nblk + KH - 1) / KH;           // blocks of split 0 (the most)
  // the last block, if partial, and whether it is this split's
  const int kb_last = nblk - 1;
  const bool has_partial = (Nk % BN) != 0 && (kb_last % KH) == splitu;

  // ---- Q^T operand (B of the score product): query l32, dims 16 ks + 8 hi;
  // dims 40-47 hold the mask weight -2^15 (dim 40) and zeros.  The scale
  // stays out of the 16-bit operand (but see fold_q).
  s8v qf[3];
  load_q_operand<TR>(qf, qh, lay.q.row, qbase + l32, hi, Nq);
  // the fp16 fast path after the first tile: Q scaled by c and rounded to
  // fp16, dim 41 = -mr (mr itself an fp16 value, so the reference is exact);
  // true if a scaled element of the query leaves fp16's finite range
  auto fold_q = [&](float mr) __attribute__((always_inline)) {
    typedef _Float16 h8v __attribute__((ext_vector_type(8)));
    float big = 0.f;
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      h8v x = __builtin_bit_cast(h8v, qf[ks]);
      float bk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = (float)x[e] * c;
        bk = __builtin_fmaxf(bk, __builtin_fabsf(y));
        x[e] = (_Float16)y;
      }
      big = (ks < 2 || !hi) ? __builtin_fmaxf(big, bk) : big;  // dims 0-39 only
      if (ks == 2) {
        h8v m = __builtin_bit_cast(h8v, (s8v){(short)TR::kMinus2p15, 0, 0, 0, 0, 0, 0, 0});
        m[1] = (_Float16)(-mr);
        x = hi ? m : x;  // lanes hi = 1 hold dims 40-47
      }
      qf[ks] = __builtin_bit_cast(s8v, x);
    }
    return !(big < 65504.f);
  };

  // ---- direct-load plan of this wave: jobs qg, qg + QG, ... of the 13 per
  // block (7 K loads, then 6 V loads), each 64 chunks of 16 bytes
  Dma<QG> dma;
#pragma unroll
  for (int r = 0; r < C::MAXJ; ++r) {
    const int j = qgu + QG * r;
    dma.voff[r] = 0x7FFFFFF0;  // padding job: out of range, zeros into the padding area
    dma.act[r] = true;
    if (j < KJOBS) {
      const int p = 64 * j + lane, row = p / KCH, ch = p - row * KCH;
      dma.act[r] = ch < 5;
      dma.voff[r] = (row * krs + ch * 8) * 2;
    } else if (j < NJOBS) {
      const int p = 64 * (j - KJOBS) + lane, grp = p / VGRP, rem = p - grp * VGRP, ch = rem >> 2;
      dma.act[r] = ch < 5;
      dma.voff[r] = ((4 * grp + (rem & 3)) * vrs + ch * 8) * 2;
    }
  }
  // the last block, if partial: K mask chunk 1.0 for its keys past Nk
  auto mask_partial = [&](int b) __attribute__((always_inline)) {
    if (has_partial && KH * b + splitu == kb_last && qgu == QG - 1) {
      const int key = (KH * b + splitu) * BN + lane;
      if (key >= Nk)
        lds_store16(ring + (b % NBUF) * SLOT + lane * KPITCH + 80, TR::kOne, 0, 0, 0);
    }
  };
  // issue the direct loads of local block b into its slot (and its mask chunks)
  auto issue = [&](int b, bool with_mask) __attribute__((always_inline)) {
    const int key0 = (KH * b + splitu) * BN;
    const unsigned kbytes = Nk > key0 ? ((unsigned)(Nk - key0 - 1) * (unsigned)krs + D) * 2u : 0u;
    const unsigned vbytes = Nk > key0 ? ((unsigned)(Nk - key0 - 1) * (unsigned)vrs + D) * 2u : 0u;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kh + (size_t)key0 * krs, kbytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vh + (size_t)key0 * vrs, vbytes);
    lds8* const sl = ring + (b % NBUF) * SLOT;
#pragma unroll
    for (int r = 0; r < C::MAXJ; ++r) {
      // the job's source and slot chunk chosen by wave-uniform selects, not branches
      const int j = qgu + QG * r;
      const bool isv = j >= KJOBS && j < NJOBS;
      lds8* const dst = j < NJOBS ? sl + (j < KJOBS ? 1024 * j : KBYTES + 1024 * (j - KJOBS)) : smem + DUMMY;
      if (dma.act[r]) dma16(isv ? vr : kr, dst, dma.voff[r]);
    }
    if (with_mask) mask_partial(b);
  };

  // ---- per-lane LDS offsets within a slot
  // K (A operand of the score product): key row 32 t + l32, chunk 2 ks + hi
  // (ks = 2, hi = 1 is the mask chunk)
  const int offK = l32 * KPITCH + hi * 16;
  // V^T (A operand of the PV product) through ds_read_b64_tr_b16: in each
  // 16-lane group the addressing lane a names key (group key base) + a / 4 and
  // dims base + 4 (a % 4), base = 16 (group % 2) + 32 mt; the key base of a
  // read is 32 t + 16 s + 8 e + 4 hi (t tile, s K step, e half of the 8 keys)
  int offV;
  {
    const int a = lane & 15, gsub = (lane >> 4) & 1;
    const int dim = 16 * gsub + 4 * (a & 3);
    offV = KBYTES + 16 * (VGRP * hi + 4 * (dim >> 3) + (a >> 2)) + 8 * ((dim >> 2) & 1);
  }
  // V^T rows 32-47 (A operand of the 16x16x32 products): 16-lane group g
  // holds keys base(g) + 0..3 and base(g) + 8..11 of a 32-key tile, base =
  // 0, 16, 4, 20 (the key order of P after the swaps); addressing lane a
  // names key base + a / 4 (+ 8 in the second read), dims 32 + 4 (a % 4):
  // chunk 4 (dims 32-39) or chunk 5 (1.0 at dim 40, then zeros)
  int offW;
  {
    const int a = lane & 15, g = lane >> 4;
    const int grp = (g & 1) * 4 + (g >> 1);  // base / 4
    offW = KBYTES + 16 * (VGRP * grp + 4 * (4 + ((a & 3) >> 1)) + (a >> 2)) + 8 * (a & 1);
  }

  // ---- building blocks of the pipeline
  // scores of tile t (0/1) of the block in slot sl: S^T, 32 keys x 32 queries
  auto qk = [&](const lds8* sl, int t) __attribute__((always_inline)) {
    const lds8* p = sl + offK + t * 32 * KPITCH;
    f16v s = TR::mma32(lds_read_b128(p), qf[0], (f16v){});
    s = TR::mma32(lds_read_b128(p + 32), qf[1], s);
    s = TR::mma32(lds_read_b128(p + 64), qf[2], s);
    return s;
  };
  // O^T += V^T P^T over tile t of the block in slot sl (P packed: pp[2 s + i]):
  // dims 0-31 in o0 (32x32 layout), dims 32-47 in oa (queries 0-15) and ob
  // (queries 16-31), 16x16 layout: lane (n, r) holds dims 32 + 4 r .. + 3 of
  // query n (+ 16 in ob)
  f16v o0 = (f16v){};
  f4v oa = (f4v){}, ob = (f4v){};
  float oscale = 1.f;  // the exact pass: factor O takes to the current reference
  auto pv = [&](const lds8* sl, int t, const uint32_t (&pp)[8], bool exact) __attribute__((always_inline)) {
    if (exact) {
      // the previous tile's 16x16x32 results may still be in flight: wait
      // them out (the compiler does not see the products as such)
      asm volatile("s_nop 7\n\ts_nop 7" : "+v"(oa), "+v"(ob));
      // the factor is per query l32; oa holds query lane % 16, ob 16 + lane % 16
      const float sa = __shfl(oscale, lane & 15), sb = __shfl(oscale, 16 + (lane & 15));
      o0 *= oscale;
      oa *= sa;
      ob *= sb;
      oscale = 1.f;
    }
    const s4v w0 = lds_tr(sl + offW + 16 * VGRP * 8 * t), w1 = lds_tr(sl + offW + 16 * VGRP * (8 * t + 2));
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const s8v bop = __builtin_bit_cast(s8v, (uint4){pp[4 * s], pp[4 * s + 1], pp[4 * s + 2], pp[4 * s + 3]});
      const int kofs = 16 * VGRP * (8 * t + 4 * s);
      const s4v a0 = lds_tr(sl + offV + kofs), a1 = lds_tr(sl + offV + kofs + 16 * VGRP * 2);
      o0 = TR::mma32((s8v){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}, bop, o0);
    }
    // P re-laid out for the 16x16x32 products: x[0..3] then holds queries
    // 0-15 and x[4..7] queries 16-31, keys base(g) + 0..3, + 8..11 per group
    const auto r0 = __builtin_amdgcn_permlane16_swap(pp[0], pp[4], false, false);
    const auto r1 = __builtin_amdgcn_permlane16_swap(pp[1], pp[5], false, false);
    const auto r2 = __builtin_amdgcn_permlane16_swap(pp[2], pp[6], false, false);
    const auto r3 = __builtin_amdgcn_permlane16_swap(pp[3], pp[7], false, false);
    const s8v wop = (s8v){w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
    mma16_acc<TR>(wop, __builtin_bit_cast(s8v, (uint4){r0[0], r1[0], r2[0], r3[0]}), oa);
    mma16_acc<TR>(wop, __builtin_bit_cast(s8v, (uint4){r0[1], r1[1], r2[1], r3[1]}), ob);
  };
  float mref = 0.f, mtrue = -INFINITY, lsum = 0.f;
  // the folded fast path holds for references within +-64 and a scaled query
  // within fp16's range: beyond, the fp16 reference loses range and Q's
  // rounding weighs more, or a score comes out infinite (a key's true score
  // can then still weigh), so the workgroup redoes its rows on the exact
  // pass, which keeps the scale in fp32
  bool fold_bad = false;
  // P of a score tile against mref, rounded and packed (the fast path)
  // (folded: the scores are already c s - mref)
  auto expo = [&](const f16v& s, uint32_t (&pp)[8], bool folded) __attribute__((always_inline)) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(folded ? s[i] : __builtin_fmaf(s[i], c, -mref));
#pragma unroll
    for (int i = 0; i < 8; ++i) pp[i] = TR::pack2(p[2 * i], p[2 * i + 1]);
    if constexpr (kValuSum) {
#pragma unroll
      for (int i = 0; i < 16; ++i) lsum += p[i];
    }
  };
  auto tile_max = [&](const f16v& s) __attribute__((always_inline)) {
    float m = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = __builtin_fmaxf(m, s[i]);
    return pair_max32(m);  // both lanes of a query
  };
  // the exact online form: move the reference to the running max first
  // (O and the fp32 sum scaled to it), then P
  auto expo_exact = [&](const f16v& s, uint32_t (&pp)[8]) __attribute__((always_inline)) {
    const float mn = __builtin_fmaxf(mref, tile_max(s) * c);
    const float alpha = __builtin_amdgcn_exp2f(mref - mn);
    oscale = alpha;  // O moves to the new reference in the next pv, before P of this tile

    lsum *= alpha;
    mref = mn;
    expo(s, pp, false);
  };

  if (tid == 0) redo_flag = 0;

  // ---- one pass over the keys; EXACT selects the online reference
  // (a plain lambda inlined at its two call sites with a constant argument,
  // so that every test of `exact` folds away)
  auto run = [&](bool exact) __attribute__((always_inline)) {
    if constexpr (kFold) {
      if (exact) load_q_operand<TR>(qf, qh, lay.q.row, qbase + l32, hi, Nq);  // unscaled again
    }
    o0 = (f16v){};
    oa = (f4v){};
    ob = (f4v){};
    oscale = 1.f;
    lsum = 0.f;
    mtrue = -INFINITY;
    const int npre = nb < NBUF ? nb : NBUF, nfirst = npre < 1 ? npre : 1;
    // block 0's direct loads go out first: they write none of the constant
    // chunks below (its mask chunks, if it is the partial block, follow them)
    if (nfirst > 0) issue(0, false);
    // V ones chunks and K mask chunks of every slot of this split
    for (int e = tid % C::HT; e < NBUF * BN; e += C::HT) {
      lds8* sl = ring + (e / BN) * SLOT;
      const int key = e % BN;
      lds_store16(sl + KBYTES + 16 * (VGRP * (key >> 2) + 20 + (key & 3)), TR::kOne, 0, 0, 0);
      lds_store16(sl + key * KPITCH + 80, kFold ? (uint32_t)TR::kOne << 16 : 0u, 0, 0, 0);
    }
    wait_lds();
    barrier();  // every constant chunk is written before a partial block's mask chunks
    // block 0 lands before the pass starts; blocks 1-3 are issued only then
    // (with every workgroup of the chip starting at once, the first block
    // would otherwise queue behind the others' bytes), and block 1 is waited
    // for after the first block's two score tiles
    if (nfirst > 0) mask_partial(0);
    wait_vm<0>();
    wait_lds();
    barrier();
    for (int b = nfirst; b < npre; ++b) issue(b, true);

    uint32_t pa[8], pb[8];
    f16v s1 = (f16v){};
    if (nb > 0) {
      // tile 0: its exact max is the reference (keys past Nk score -2^15 scale)
      const f16v s0 = qk(ring, 0);
      if constexpr (kPV) {
        const int row = qbase + l32;
        mref = row < Nq ? ml[((size_t)head * Nq + row) * 2] * kLog2e : 0.f;
      } else {
        const float m0 = tile_max(s0) * c;
        // fp16 P: the reference sits kHeadroom above the first tile's max, so
        // that scores up to 16 + kHeadroom above it stay finite
        mref = (!exact && TR::kPackedMax) ? m0 + kHeadroom : m0;
        if (exact || kML) mtrue = m0;
        if constexpr (kFold) {
          if (!exact) {
            mref = (float)(_Float16)mref;
            const bool overflow = fold_q(mref);
            fold_bad = overflow || !(__builtin_fabsf(mref) <= 64.f);
          }
        }
      }
      s1 = qk(ring, 1);
      expo(s0, pa, false);
    }
    // block 1 lands before the first body reads it (blocks 2, 3 may be in flight)
    if (npre >= 4)
      wait_vm<2 * C::MAXJ>();
    else if (npre == 3)
      wait_vm<C::MAXJ>();
    else
      wait_vm<0>();
    wait_lds();
    barrier();
    // one tile step: P of `cur` into `pout`, scores of the next tile into
    // `snext` (when there is one), PV of the previous tile (`pin`)
    auto step = [&](const lds8* ks, int kt, const lds8* vs, int vt, const f16v& cur, f16v& snext,
                    const uint32_t (&pin)[8], uint32_t (&pout)[8], bool has_next) __attribute__((always_inline)) {
      if (has_next) snext = qk(ks, kt);
      pv(vs, vt, pin, exact);
      if (exact) {
        expo_exact(cur, pout);
      } else {
        if constexpr (kML) mtrue = __builtin_fmaxf(mtrue, tile_max(cur) * c);
        expo(cur, pout, kFold);
      }
    };
    // full bodies: tiles 2b+1 and 2b+2, scores of block b+1, PV of block b
    auto body = [&](int b) __attribute__((always_inline)) {
      const lds8* ks = ring + ((b + 1) % NBUF) * SLOT;
      const lds8* vs = ring + (b % NBUF) * SLOT;
      f16v s2;
      step(ks, 0, vs, 0, s1, s2, pa, pb, true);
      step(ks, 1, vs, 1, s2, s1, pb, pa, true);
    };
    int b = 0;
    // while two blocks are in flight: wait for the older one (block b+2)
    for (; b + 3 < nb; ++b) {
      body(b);
      wait_vm<C::MAXJ>();
      wait_lds();
      barrier();
      if (b + NBUF < nb) issue(b + NBUF, true);
    }
    for (; b < nb - 1; ++b) {
      body(b);
      wait_vm<0>();
      wait_lds();
      barrier();
    }
    if (nb > 0) {
      // the last block: PV of its two tiles
      const lds8* vs = ring + ((nb - 1) % NBUF) * SLOT;
      f16v unused;
      step(vs, 0, vs, 0, s1, unused, pa, pb, false);
      pv(vs, 1, pb, exact);
      barrier();
    }
    // a split with fewer blocks meets the other's barriers
    for (int e = nb > 0 ? nb : 0; e < niter; ++e) barrier();
    if (exact) mtrue = mref;
  };

  run(false);
  // the row sum (the loop above may end on either of two branches: mfma_settled)
  float lrow = row_sum(mfma_settled(oa[0]), mfma_settled(ob[0]), l32);
  if constexpr (!kPV) {
    // a row whose sum left the fast path's range is recomputed by all waves
    if (nb > 0 && __any(!(lrow < kSumLimit) || fold_bad)) redo_flag = 1;
    wait_lds();
    barrier();
    if (redo_flag) {
      barrier();
      run(true);
      lrow = row_sum(mfma_settled(oa[0]), mfma_settled(ob[0]), l32);
    }
  }
  if (nb == 0) {
    mref = -INFINITY;  // this split saw no key: it must not weigh in the merge
    mtrue = -INFINITY;
  }
  float lr = kValuSum ? pair_sum32(lsum) : lrow;
  // dims 32 + 4 hi .. + 3 of query l32, from lane (l32 % 16) + 16 hi of oa
  // or ob: from here on every value of a lane belongs to query l32
  float d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float da = __shfl(oa[i], (l32 & 15) + 16 * hi), db = __shfl(ob[i], (l32 & 15) + 16 * hi);
    d[i] = l32 < 16 ? da : db;
  }

  // ---- merge the key splits: split 1 hands (m, O, l) to split 0 through LDS
  wait_lds();
  barrier();  // every wave is done with the ring
  float* const ex = (float*)(smem_) + qg * C::XN * 64 + lane;
  if (split > 0) {
    ex[0] = mref;
    ex[64] = mtrue;
    ex[128] = lr;
    ex[192] = lrow;
#pragma unroll
    for (int i = 0; i < 16; ++i) ex[(4 + i) * 64] = o0[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) ex[(20 + i) * 64] = d[i];
  }
  wait_lds();
  barrier();
  if (split > 0) return;
  {
    const float mB = ex[0], mtB = ex[64], lrB = ex[128], lrowB = ex[192];
    // a split that saw no key holds (-inf, 0): it contributes nothing
    const float M = kPV ? mref : __builtin_fmaxf(mref, mB);
    const float fA = kPV ? 1.f : __builtin_amdgcn_exp2f(mref - M);
    const float fB = kPV ? 1.f : __builtin_amdgcn_exp2f(mB - M);
    // explicit FMAs: the contraction of the merge is fixed
#pragma unroll
    for (int i = 0; i < 16; ++i) o0[i] = __builtin_fmaf(o0[i], fA, ex[(4 + i) * 64] * fB);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = __builtin_fmaf(d[i], fA, ex[(20 + i) * 64] * fB);
    lr = __builtin_fmaf(lr, fA, lrB * fB);
    lrow = __builtin_fmaf(lrow, fA, lrowB * fB);
    mtrue = __builtin_fmaxf(mtrue, mtB);
    mref = M;
  }
  const float l = lrow;  // the merged row sum
  const int row = qbase + l32;
  if (row >= Nq) return;
  float inv;
  if constexpr (kPV) {
    inv = 1.f / ml[((size_t)head * Nq + row) * 2 + 1];  // P was formed against the given m
  } else {
    inv = 1.f / l;
  }
  uint16_t* op = out + head_offset(lay.o, lay.H, head) + (size_t)row * lay.o.row;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint2 w;
    w.x = TR::pack2(o0[4 * i] * inv, o0[4 * i + 1] * inv);
    w.y = TR::pack2(o0[4 * i + 2] * inv, o0[4 * i + 3] * inv);
    *(uint2*)(op + 8 * i + 4 * hi) = w;
  }
  {
    uint2 w;
    w.x = TR::pack2(d[0] * inv, d[1] * inv);
    w.y = TR::pack2(d[2] * inv, d[3] * inv);
    *(uint2*)(op + 32 + 4 * hi) = w;
  }
  if constexpr (kML) {
    if (hi == 0) {
      // l was accumulated against the reference M; report it against the true max
      const float lsel = kValuSum ? lr : l;
      const float lt = lsel * __builtin_amdgcn_exp2f(mref - mtrue);
      *(float2*)(ml + ((size_t)head * Nq + row) * 2) = make_float2(mtrue / kLog2e, lt);
    }
  }
}

template <class TR, int MODE, int QG>
hipError_t launch_fa40_q(const Problem& p, long long nwg, int qtiles) {
  hipLaunchKernelGGL((fa40_kernel<TR, MODE, QG>), dim3((unsigned)nwg), dim3(fa40::Cfg<QG>::T), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v, (uint16_t*)p.out, p.ml,
                     p.lay, p.Nq, p.Nk, qtiles, (int)nwg, p.scale);
  return hipGetLastError();
}

// The widest workgroup (8 query groups) when it fills the chip; otherwise 4,
// then 2 query groups per workgroup for more workgroups.
template <class TR, int MODE>
hipError_t launch_fa40_t(const Problem& p, int cus) {
  const long long q8 = (p.Nq + 255) / 256, q4 = (p.Nq + 127) / 128, q2 = (p.Nq + 63) / 64;
  if ((long long)p.BH * q8 >= cus || (long long)p.BH * q4 > 0x7fffffffLL) {
    if ((long long)p.BH * q8 > 0x7fffffffLL) return hipErrorInvalidValue;
    return launch_fa40_q<TR, MODE, 8>(p, p.BH * q8, (int)q8);
  }
  if ((long long)p.BH * q4 >= cus) return launch_fa40_q<TR, MODE, 4>(p, p.BH * q4, (int)q4);
  return launch_fa40_q<TR, MODE, 2>(p, p.BH * q2, (int)q2);
}

template <int MODE>
hipError_t launch_fa40_m(const Problem& p, int cus) {
  return p.dt == ATTN_BF16 ? launch_fa40_t<BF16, MODE>(p, cus) : launch_fa40_t<F16, MODE>(p, cus);
}

}  // namespace

hipError_t launch_fa40_flash(const Problem& p, int cus) {
  return p.ml ? launch_fa40_m<kModeFlashML>(p, cus) : launch_fa40_m<kModeFlash>(p, cus);
}
hipError_t launch_fa40_pv(const Problem& p, int cus) { return launch_fa40_m<kModePV>(p, cus); }

}  // namespace attn
