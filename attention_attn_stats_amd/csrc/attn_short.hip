// Matrix-core FlashAttention for short key ranges (at most 256 keys at head
// dims 80 and 160, 384 at 40): the UNet's cross-attention over the 77 text
// tokens and the self-attention of its deepest levels (64 and 256 positions).
//
// Method: "Speed Is All You Need: On-Device Acceleration of Large Diffusion
// Models via GPU-Aware Optimizations" (Chen et al.), news write-up, section on
// improving attention efficiency: O = softmax(scale Q K^T) V in one pass, the
// key range cut into blocks that are reduced separately and merged (the
// block-split reduction), here one block per wave.
//
// With so few keys a launch is bound by latency, not by bandwidth or the
// matrix cores: every load of a wave (its queries, its keys, its values) is
// issued at once at the start, each wave holds all scores of its block in
// registers (so the row max is exact before any exponential and nothing is
// rescaled), and the only synchronisation is one workgroup barrier before the
// merge of the key splits.
//
//   * a wave owns 16 queries and a block of up to 16 NKT keys (NKT 16-key
//     tiles); S^T = K Q^T on 16x16x32 MFMAs, both operands read straight from
//     memory in operand layout (lane (G, li): row li, elements 8G .. 8G+7 of
//     a 32-element step).  Lane (G, li) then holds keys 4G .. 4G+3 of every
//     tile for query li.
//   * those are exactly the B operand of O^T += V^T P^T on 16x16x32 MFMAs for
//     a 32-key step made of tiles 2j and 2j+1, taken in the key order
//     (4G .. 4G+3, 16+4G .. 16+4G+3): no exchange between lanes.  V^T comes
//     from the wave's own LDS copy of its V rows through ds_read_b64_tr_b16
//     in that order.
//   * d = 40 pads the PV product to 48 rows; LDS column 40 of V holds 1.0 so
//     row 40 of O^T is the row sum l of the same rounded P.
//   * the W = 4 waves of a workgroup are 4 / kspl query groups x kspl key
//     splits; splits merge (m, l, O) through LDS, each wave finishing a share
//     of the 16-dim tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>

#include "attn_internal.h"
#include "mfma_common.h"

namespace attn {
namespace {

template <int D>
struct ShortShape {
  static constexpr int KS = (D + 31) / 32;      // 32-dim steps of S^T = K Q^T
  static constexpr int MT = (D + 15) / 16;      // 16-dim tiles of O^T
  static constexpr bool kOnes = (D % 16) != 0;  // LDS column D of V holds 1.0 -> O^T row D = l
  static constexpr bool kPadQK = (D % 32) != 0; // the last 32-dim step reaches past d
  // LDS row pitch of V (16-bit elements): ds_read_b64_tr_b16 takes 4 rows x
  // 32 bytes per 16 lanes, 16 consecutive rows per wave; a pitch of 24 or 40
  // words mod 64 puts every 8 consecutive rows in distinct banks
  static constexpr int PV = D == 40 ? 48 : (D == 80 ? 80 : D + 16);
  static constexpr int NKT = D == 40 ? 6 : 4;   // most 16-key tiles per wave
  static constexpr int W = 4;                   // waves per workgroup
  static constexpr int VCH = D / 8;             // 16-byte chunks per V row
  static constexpr int KEYS = W * NKT * 16;     // longest key range
  // V rows the PV steps of a wave with TPW tiles read (whole 32-key steps)
  static constexpr int vrows(int tpw) { return 32 * ((tpw + 1) / 2); }
  // bytes of LDS per wave: its V rows, later its (O^T, m, l, l reported) for the merge
  static constexpr int region(int tpw) {
    const int a = vrows(tpw) * PV * 2, b = MT * 1024 + 3 * 64;
    return ((a > b ? a : b) + 15) / 16 * 16;
  }
  static_assert(D % 8 == 0, "head dim must be a multiple of 8");
};

// Reductions over the four 16-lane rows (lanes li, li + 16, li + 32, li + 48).
// A swap of a value with itself is written as inline asm (the builtin's two
// results would be taken as interchangeable and the reduction folded away);
// the s_nop covers the wait states after a vector-ALU write of the input.
template <class Op>
__device__ __forceinline__ float row16_reduce(float x, Op op) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 4\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  x = op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  a = __builtin_bit_cast(uint32_t, x);
  b = a;
  asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float row16_max(float x) {
  return row16_reduce(x, [](float a, float b) { return __builtin_fmaxf(a, b); });
}
__device__ __forceinline__ float row16_sum(float x) {
  return row16_reduce(x, [](float a, float b) { return a + b; });
}

// One workgroup: 4 / kspl query groups of 16 queries x kspl key splits of
// TPW 16-key tiles (grid: x = query tile, y = head in batch, z = batch).  Everything a wave
// indexes by is wave-uniform scalar work, and its loads, LDS accesses and
// stores use one per-lane address each plus immediate offsets: with so little
// work per wave, the count of instructions it issues sets the time.
template <class TR, int D, int TPW, int KSPL, bool kML>
__global__ __launch_bounds__(256) void short_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
                                                    float* __restrict__ ml, const Layout lay, int Nq, int Nk,
                                                    float scale) {
  using S = ShortShape<D>;
  constexpr int KS = S::KS, MT = S::MT, PV = S::PV, VCH = S::VCH;
  constexpr int VROWS = S::vrows(TPW), REGION = S::region(TPW);
  // l from the fp32 sum of the unrounded P: where no ones column exists, and
  // for a reported l in bf16 (its 8-bit rounding is too coarse for it)
  constexpr bool kValuSum = !S::kOnes || (kML && !TR::kRoundedSumOk);
  constexpr int kNone = 0x7FFFFFF0;  // an offset past every resource: reads zero
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::W * REGION];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4, li = lane & 15;
  constexpr int kspl = KSPL, ksh = KSPL == 4 ? 2 : (KSPL == 2 ? 1 : 0);
  static_assert(KSPL == 1 || KSPL == 2 || KSPL == 4, "key splits: 1, 2 or 4");
  const int split = wave & (kspl - 1), qg = wave >> ksh;
  const int head = blockIdx.z * lay.H + blockIdx.y;  // batch-major head index (of ml)
  const long long qh = blockIdx.z * lay.q.batch + blockIdx.y * lay.q.head, kh = blockIdx.z * lay.k.batch + blockIdx.y * lay.k.head;
  const long long vh = blockIdx.z * lay.v.batch + blockIdx.y * lay.v.head, oh = blockIdx.z * lay.o.batch + blockIdx.y * lay.o.head;
  const int q0 = (((int)blockIdx.x << (2 - ksh)) + qg) << 4;
  const int kb = split * 16 * TPW;  // first key of this wave
  const float c = scale * kLog2e;
  const int qrs = lay.q.row, krs = lay.k.row, vrs = lay.v.row;
  // lanes whose 8 elements of the last 32-dim step lie past d read nothing
  // there (zeros in Q and in K: padding between rows may hold anything)
  const bool padlane = S::kPadQK && 32 * (KS - 1) + 8 * G >= D;

  // ---- every load at once.  Q (B operand of S^T): row q0 + li, dims 8G +
  // 32 ks; rows past Nq read as zero
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(q + qh, ((unsigned)(Nq - 1) * (unsigned)qrs + D) * 2u);
  const unsigned qoff = ((unsigned)(q0 + li) * (unsigned)qrs + 8 * G) * 2u;
  s8v qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = __builtin_bit_cast(s8v, load16(qr, (ks == KS - 1 && padlane) ? kNone : (int)(qoff + 64 * ks)));
  // K (A operand): key kb + 16 t + li, dims 8G + 32 ks; the resources run
  // from this wave's first key to key Nk, so keys past Nk read as zero
  const unsigned kbytes = Nk > kb ? ((unsigned)(Nk - kb - 1) * (unsigned)krs + D) * 2u : 0u;
  const unsigned vbytes = Nk > kb ? ((unsigned)(Nk - kb - 1) * (unsigned)vrs + D) * 2u : 0u;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + kh + (size_t)kb * krs, kbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + vh + (size_t)kb * vrs, vbytes);
  const unsigned koff = ((unsigned)li * (unsigned)krs + 8 * G) * 2u;
  s8v kf[TPW][KS];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[t][ks] = __builtin_bit_cast(
          s8v, load16(kr, (ks == KS - 1 && padlane) ? kNone : (int)(koff + (unsigned)(32 * t) * (unsigned)krs + 64 * ks)));
  // V rows of the block, as 16-byte chunks in row-major order: load j takes
  // chunks 64 j .. 64 j + 63, one contiguous kilobyte of a dense tensor (the
  // fastest pattern for a CU's load path).  Five loads cover RB = 320 / VCH
  // rows, so a lane's (row, chunk) of load 5 m + n is (R_n + RB m, C_n).
  // Rows past the wave's tiles or past Nk read as zeros (their P are zero,
  // and 0 * a stale non-finite LDS value would not be).
  constexpr int RB = 320 / VCH, DROWS = 16 * TPW;
  constexpr int VJ = (DROWS * VCH + 63) / 64;  // loads with data
  static_assert(320 % VCH == 0, "five loads cover whole rows");
  int vgo[5], vlo[5], vrn[5];                   // global byte offset, LDS element offset, row of load n
#pragma unroll
  for (int n = 0; n < 5; ++n) {
    const int idx = 64 * n + lane, r = idx / VCH, col = idx - r * VCH;
    vrn[n] = r;
    vgo[n] = (int)(((unsigned)r * (unsigned)vrs + 8 * col) * 2u);
    vlo[n] = r * PV + 8 * col;
  }
  uint4 stg[VJ];
#pragma unroll
  for (int j = 0; j < VJ; ++j) {
    const int n = j % 5, m = j / 5;
    const bool whole = RB * m + RB <= DROWS;  // every row of this period has data
    const int off = vgo[n] + (int)((unsigned)(RB * m) * (unsigned)vrs * 2u);
    stg[j] = load16(vr, whole || vrn[n] + RB * m < DROWS ? off : kNone);
  }

  // No load is issued once the products have started: a load landing in a
  // register that an in-flight MFMA has yet to read as its accumulator input
  // corrupts single lanes (seen on MI355X as single wrong query rows).
  __builtin_amdgcn_sched_barrier(0);

  // ---- scores, tile t: keys kb + 16 t + 4G + i (i = 0..3), query q0 + li
  f4v sc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    sc[t] = (f4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc[t] = TR::mma16(kf[t][ks], qf[ks], sc[t]);
  }
  // keys past Nk: -inf, by selects without a branch (a branch between the
  // products and these first reads of their results lets the compiler count
  // too few wait states on one of the paths)
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[t][i] = kb + 16 * t + 4 * G + i < Nk ? sc[t][i] : -INFINITY;
  // exact max of the block (scale > 0: the max of the raw scores), in exp2
  // units; a split past every key keeps -inf and weighs nothing in the merge
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    mx = __builtin_fmaxf(__builtin_fmaxf(mx, __builtin_fmaxf(sc[t][0], sc[t][1])), __builtin_fmaxf(sc[t][2], sc[t][3]));
  const float M2 = row16_max(mx) * c;
  const bool any = kb < Nk;  // wave-uniform
  // P = exp2(c s - M2), rounded to 16 bits, packed as the B operands of the PV steps
  float lv = 0.f;
  uint32_t pp[TPW + 1][2];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = any ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][i], c, -M2)) : 0.f;
    if constexpr (kValuSum) lv += (p[0] + p[1]) + (p[2] + p[3]);
    pp[t][0] = TR::pack2(p[0], p[1]);
    pp[t][1] = TR::pack2(p[2], p[3]);
  }
  pp[TPW][0] = pp[TPW][1] = 0u;

  // ---- V block into this wave's LDS region (only this wave reads it); rows
  // DROWS .. VROWS - 1 (an odd tile count) as zeros
  uint16_t* const vs = (uint16_t*)(smem + wave * REGION);
#pragma unroll
  for (int j = 0; j < VJ; ++j) {
    const int n = j % 5, m = j / 5;
    if (RB * m + RB <= VROWS || vrn[n] + RB * m < VROWS) *(uint4*)(vs + vlo[n] + RB * m * PV) = stg[j];
  }
  if constexpr (VROWS > DROWS) {
    constexpr int ZCH = (VROWS - DROWS) * VCH;  // chunks of zero rows
#pragma unroll
    for (int z = lane; z < ZCH; z += 64) {
      const int r = DROWS + z / VCH, col = z - (z / VCH) * VCH;
      *(uint4*)(vs + r * PV + 8 * col) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // columns D .. PV-1: 1.0 in column D (the row-sum dim), zeros after it
  if constexpr (S::kOnes) {
    for (int r = lane; r < VROWS; r += 64) *(uint4*)(vs + r * PV + D) = make_uint4(TR::kOne, 0u, 0u, 0u);
  }
  // (a wave's LDS operations complete in order: its reads below see its writes)

  // ---- O^T += V^T P^T, lane (G, li): dims 16 mt + 4G + i, query li
  f4v o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = (f4v){0.f, 0.f, 0.f, 0.f};
  // (every V operand read before the first product: no load among them)
  const uint16_t* const va = vs + (4 * G + (li >> 2)) * PV + 4 * (li & 3);
  s8v vop[(TPW + 1) / 2][MT];
#pragma unroll
  for (int j = 0; j < (TPW + 1) / 2; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const s4v v0 = lds_read_tr16(va + 32 * j * PV + 16 * mt);
      const s4v v1 = lds_read_tr16(va + (32 * j + 16) * PV + 16 * mt);
      vop[j][mt] = (s8v){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < (TPW + 1) / 2; ++j) {
    const s8v pb = __builtin_bit_cast(s8v, (uint4){pp[2 * j][0], pp[2 * j][1], pp[2 * j + 1][0], pp[2 * j + 1][1]});
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = TR::mma16(vop[j][mt], pb, o[mt]);
  }

  // ---- row sums: the normaliser and the reported l
  float lnorm, lrep;
  if constexpr (kValuSum) lv = row16_sum(lv);
  if constexpr (S::kOnes) {
    constexpr int GL = (D % 16) / 4, IL = D % 4;
    lnorm = __shfl(o[MT - 1][IL], GL * 16 + li);
  } else {
    lnorm = lv;
  }
  lrep = kValuSum ? lv : lnorm;

  const int row = q0 + li;
  const bool rowok = row < Nq;
  uint16_t* const op = out + oh + (size_t)(rowok ? row : 0) * lay.o.row + 4 * G;
  auto store_tile = [&](int mt, f4v x, float inv) {
    if (rowok && (!S::kOnes || mt < MT - 1 || 16 * mt + 4 * G < D)) {
      uint2 w;
      w.x = TR::pack2(x[0] * inv, x[1] * inv);
      w.y = TR::pack2(x[2] * inv, x[3] * inv);
      *(uint2*)(op + 16 * mt) = w;
    }
  };
  auto store_ml = [&](float m2, float l) {
    if (kML && G == 0 && rowok) *(float2*)(ml + ((size_t)head * Nq + row) * 2) = make_float2(m2 / kLog2e, l);
  };

  if constexpr (KSPL == 1) {
    const float inv = __builtin_amdgcn_rcpf(lnorm);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) store_tile(mt, o[mt], inv);
    store_ml(M2, lrep);
    return;
  }

  // ---- merge of the key splits: every wave leaves (O^T, m, l) in its region
  // (after its own V reads, in order), then finishes the tiles mt = split,
  // split + kspl, ... of its query group from all splits
  {
    float* const x = (float*)(smem + wave * REGION);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *(f4v*)(x + (mt * 64 + lane) * 4) = o[mt];
    if (G == 0) {
      x[MT * 256 + li] = any ? M2 : -INFINITY;
      x[MT * 256 + 16 + li] = lnorm;
      x[MT * 256 + 32 + li] = lrep;
    }
  }
  __syncthreads();
  const unsigned char* const x0 = smem + (wave - split) * REGION;  // split 0 of this query group
  float M = -INFINITY;
#pragma unroll
  for (int t = 0; t < S::W; ++t)
    if (t < kspl) M = __builtin_fmaxf(M, ((const float*)(x0 + t * REGION))[MT * 256 + li]);
  float f[S::W], L = 0.f, Lr = 0.f;
#pragma unroll
  for (int t = 0; t < S::W; ++t) {
    f[t] = 0.f;
    if (t < kspl) {
      const float* const xt = (const float*)(x0 + t * REGION);
      f[t] = __builtin_amdgcn_exp2f(xt[MT * 256 + li] - M);
      L = __builtin_fmaf(xt[MT * 256 + 16 + li], f[t], L);
      Lr = __builtin_fmaf(xt[MT * 256 + 32 + li], f[t], Lr);
    }
  }
  const float inv = __builtin_amdgcn_rcpf(L);
  for (int mt = split; mt < MT; mt += kspl) {
    f4v acc = (f4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < S::W; ++t) {
      if (t < kspl) {
        const f4v y = *(const f4v*)((const float*)(x0 + t * REGION) + (mt * 64 + lane) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(y[i], f[t], acc[i]);
      }
    }
    store_tile(mt, acc, inv);
  }
  if (split == 0) store_ml(M, Lr);
}

// Shared form, for many queries per head over at most 96 keys (the text
// cross-attention): the workgroup's 8 waves (QPW groups of 16 queries each,
// all keys) stage K and V once in LDS and share them; a wave that loaded its
// own copies would send the same bytes through the CU's load path once per
// 16 queries.  A wave's K and V operands serve all its query groups, and its
// fixed work (addressing, reductions) is spread over them.  Grid: x = block
// of 16 QPW 8 queries, y = head in batch, z = batch.
constexpr int kSharedW = 8;                 // waves per workgroup
constexpr int kSharedTiles = 6;             // most 16-key tiles (96 keys)
template <int D>
constexpr int shared_pk() { return D == 40 ? 40 : D + 8; }  // K row pitch: 16 rows per ds_read_b128 in distinct banks
template <int D>
constexpr int shared_qpw() { return D == 40 ? 2 : 1; }      // query groups per wave (registers allow two at d = 40)

template <class TR, int D, int TPW, bool kML>
__global__ __launch_bounds__(64 * kSharedW) void short_shared_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, float* __restrict__ ml, const Layout lay, int Nq, int Nk, float scale) {
  using S = ShortShape<D>;
  constexpr int KS = S::KS, MT = S::MT, PV = S::PV, VCH = S::VCH, PK = shared_pk<D>(), QPW = shared_qpw<D>();
  constexpr int W = kSharedW, T = 64 * W;
  constexpr int KROWS = 16 * TPW, VROWS = S::vrows(TPW);
  constexpr bool kValuSum = !S::kOnes || (kML && !TR::kRoundedSumOk);
  constexpr int kNone = 0x7FFFFFF0;
  __shared__ __attribute__((aligned(16))) uint16_t smem[KROWS * PK + VROWS * PV];
  uint16_t* const ks_ = smem;
  uint16_t* const vs_ = smem + KROWS * PK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, li = lane & 15;
  const int head = blockIdx.z * lay.H + blockIdx.y;
  const long long qh = blockIdx.z * lay.q.batch + blockIdx.y * lay.q.head, kh = blockIdx.z * lay.k.batch + blockIdx.y * lay.k.head;
  const long long vh = blockIdx.z * lay.v.batch + blockIdx.y * lay.v.head, oh = blockIdx.z * lay.o.batch + blockIdx.y * lay.o.head;
  const int q0 = ((int)blockIdx.x * W + wave) * 16 * QPW;  // query group g: rows q0 + 16 g + li
  const float c = scale * kLog2e;
  const int qrs = lay.q.row, krs = lay.k.row, vrs = lay.v.row;
  const bool padlane = S::kPadQK && 32 * (KS - 1) + 8 * G >= D;

  // ---- every load at once: this wave's Q; the workgroup's K and V rows
  // (16-byte chunk idx = tid + T j: row idx / VCH, chunk idx % VCH); keys
  // past Nk read as zero
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(q + qh, ((unsigned)(Nq - 1) * (unsigned)qrs + D) * 2u);
  const unsigned qoff = ((unsigned)(q0 + li) * (unsigned)qrs + 8 * G) * 2u;
  s8v qf[QPW][KS];
#pragma unroll
  for (int g = 0; g < QPW; ++g)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[g][ks] = __builtin_bit_cast(
          s8v, load16(qr, (ks == KS - 1 && padlane) ? kNone : (int)(qoff + (unsigned)(16 * g) * (unsigned)qrs * 2u + 64 * ks)));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(k + kh, ((unsigned)(Nk - 1) * (unsigned)krs + D) * 2u);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(v + vh, ((unsigned)(Nk - 1) * (unsigned)vrs + D) * 2u);
  constexpr int KJ = (KROWS * VCH + T - 1) / T, VJ = (VROWS * VCH + T - 1) / T;
  uint4 kst[KJ], vst[VJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int idx = tid + T * j, r = idx / VCH, col = idx - r * VCH;
    kst[j] = load16(kr, idx < KROWS * VCH ? (int)(((unsigned)r * (unsigned)krs + 8 * col) * 2u) : kNone);
  }
#pragma unroll
  for (int j = 0; j < VJ; ++j) {
    const int idx = tid + T * j, r = idx / VCH, col = idx - r * VCH;
    // rows past the tiles (to the end of the last 32-key step) as zeros
    vst[j] = load16(vr, r < KROWS ? (int)(((unsigned)r * (unsigned)vrs + 8 * col) * 2u) : kNone);
  }
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int idx = tid + T * j, r = idx / VCH, col = idx - r * VCH;
    if (idx < KROWS * VCH) *(uint4*)(ks_ + r * PK + 8 * col) = kst[j];
  }
#pragma unroll
  for (int j = 0; j < VJ; ++j) {
    const int idx = tid + T * j, r = idx / VCH, col = idx - r * VCH;
    if (idx < VROWS * VCH) *(uint4*)(vs_ + r * PV + 8 * col) = vst[j];
  }
  if constexpr (S::kOnes) {
    // V columns D .. PV-1: 1.0 in column D (the row-sum dim), zeros after it
    for (int r = tid; r < VROWS; r += T) *(uint4*)(vs_ + r * PV + D) = make_uint4(TR::kOne, 0u, 0u, 0u);
  }
  __syncthreads();

  // ---- scores, tile t: keys 16 t + 4G + i, query q0 + 16 g + li; the K
  // operands from LDS (lanes past d in the last step: zeros, whatever lies
  // there), every one read before the first product (no load among the
  // products, as in the per-wave form)
  s8v ka[TPW][KS];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ka[t][ks] = *(const s8v*)(ks_ + (16 * t + li) * PK + 32 * ks + 8 * G);
      if (ks == KS - 1 && padlane) ka[t][ks] = (s8v){0, 0, 0, 0, 0, 0, 0, 0};
    }
  __builtin_amdgcn_sched_barrier(0);
  f4v sc[QPW][TPW];
#pragma unroll
  for (int g = 0; g < QPW; ++g)
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      sc[g][t] = (f4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sc[g][t] = TR::mma16(ka[t][ks], qf[g][ks], sc[g][t]);
    }
  // keys past Nk: -inf, by selects without a branch (as in the per-wave form)
#pragma unroll
  for (int g = 0; g < QPW; ++g)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[g][t][i] = 16 * t + 4 * G + i < Nk ? sc[g][t][i] : -INFINITY;
  float M2[QPW], lv[QPW];
  uint32_t pp[QPW][TPW + 1][2];
#pragma unroll
  for (int g = 0; g < QPW; ++g) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      mx = __builtin_fmaxf(__builtin_fmaxf(mx, __builtin_fmaxf(sc[g][t][0], sc[g][t][1])),
                           __builtin_fmaxf(sc[g][t][2], sc[g][t][3]));
    M2[g] = row16_max(mx) * c;  // Nk >= 1: finite
    lv[g] = 0.f;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[g][t][i], c, -M2[g]));
      if constexpr (kValuSum) lv[g] += (p[0] + p[1]) + (p[2] + p[3]);
      pp[g][t][0] = TR::pack2(p[0], p[1]);
      pp[g][t][1] = TR::pack2(p[2], p[3]);
    }
    pp[g][TPW][0] = pp[g][TPW][1] = 0u;
  }

  // ---- O^T += V^T P^T (every V operand read before the first product)
  const uint16_t* const va = vs_ + (4 * G + (li >> 2)) * PV + 4 * (li & 3);
  s8v vop[(TPW + 1) / 2][MT];
#pragma unroll
  for (int j = 0; j < (TPW + 1) / 2; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const s4v v0 = lds_read_tr16(va + 32 * j * PV + 16 * mt);
      const s4v v1 = lds_read_tr16(va + (32 * j + 16) * PV + 16 * mt);
      vop[j][mt] = (s8v){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
  __builtin_amdgcn_sched_barrier(0);
  f4v o[QPW][MT];
#pragma unroll
  for (int g = 0; g < QPW; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[g][mt] = (f4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < (TPW + 1) / 2; ++j)
#pragma unroll
    for (int g = 0; g < QPW; ++g) {
      const s8v pb =
          __builtin_bit_cast(s8v, (uint4){pp[g][2 * j][0], pp[g][2 * j][1], pp[g][2 * j + 1][0], pp[g][2 * j + 1][1]});
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[g][mt] = TR::mma16(vop[j][mt], pb, o[g][mt]);
    }
#pragma unroll
  for (int g = 0; g < QPW; ++g) {
    float lnorm;
    if constexpr (kValuSum) lv[g] = row16_sum(lv[g]);
    if constexpr (S::kOnes) {
      constexpr int GL = (D % 16) / 4, IL = D % 4;
      lnorm = __shfl(o[g][MT - 1][IL], GL * 16 + li);
    } else {
      lnorm = lv[g];
    }
    const float lrep = kValuSum ? lv[g] : lnorm;
    const int row = q0 + 16 * g + li;
    if (row < Nq) {
      uint16_t* const op = out + oh + (size_t)row * lay.o.row + 4 * G;
      const float inv = __builtin_amdgcn_rcpf(lnorm);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (!S::kOnes || mt < MT - 1 || 16 * mt + 4 * G < D) {
          uint2 w;
          w.x = TR::pack2(o[g][mt][0] * inv, o[g][mt][1] * inv);
          w.y = TR::pack2(o[g][mt][2] * inv, o[g][mt][3] * inv);
          *(uint2*)(op + 16 * mt) = w;
        }
      }
      if (kML && G == 0) *(float2*)(ml + ((size_t)head * Nq + row) * 2) = make_float2(M2[g] / kLog2e, lrep);
    }
  }
}

template <class TR, int D, int TPW, bool kML>
hipError_t launch_shared_k(const Problem& p) {
  constexpr int qwg = 16 * shared_qpw<D>() * kSharedW;  // queries per workgroup
  const dim3 grid((unsigned)((p.Nq + qwg - 1) / qwg), (unsigned)p.lay.H, (unsigned)(p.BH / p.lay.H));
  hipLaunchKernelGGL((short_shared_kernel<TR, D, TPW, kML>), grid, dim3(64 * kSharedW), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v, (uint16_t*)p.out, p.ml, p.lay,
                     p.Nq, p.Nk, p.scale);
  return hipGetLastError();
}

template <class TR, int D, bool kML>
hipError_t launch_shared_t(const Problem& p) {
  switch ((p.Nk + 15) / 16) {
    case 1: return launch_shared_k<TR, D, 1, kML>(p);
    case 2: return launch_shared_k<TR, D, 2, kML>(p);
    case 3: return launch_shared_k<TR, D, 3, kML>(p);
    case 4: return launch_shared_k<TR, D, 4, kML>(p);
    case 5: return launch_shared_k<TR, D, 5, kML>(p);
    case 6: return launch_shared_k<TR, D, 6, kML>(p);
    default: return hipErrorInvalidValue;
  }
}

template <class TR, int D, int TPW, int KSPL, bool kML>
hipError_t launch_short_kk(const Problem& p) {
  constexpr int qwg = 16 * (ShortShape<D>::W / KSPL);  // queries per workgroup
  const dim3 grid((unsigned)((p.Nq + qwg - 1) / qwg), (unsigned)p.lay.H, (unsigned)(p.BH / p.lay.H));
  hipLaunchKernelGGL((short_kernel<TR, D, TPW, KSPL, kML>), grid, dim3(64 * ShortShape<D>::W), 0, p.stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v, (uint16_t*)p.out, p.ml, p.lay,
                     p.Nq, p.Nk, p.scale);
  return hipGetLastError();
}
template <class TR, int D, int TPW, bool kML>
hipError_t launch_short_k(const Problem& p, int ksh) {
  switch (ksh) {
    case 0: return launch_short_kk<TR, D, TPW, 1, kML>(p);
    case 1: return launch_short_kk<TR, D, TPW, 2, kML>(p);
    case 2: return launch_short_kk<TR, D, TPW, 4, kML>(p);
    default: return hipErrorInvalidValue;
  }
}

template <class TR, int D, bool kML>
hipError_t launch_short_t(const Problem& p, int cus) {
  using S = ShortShape<D>;
  const int nt = (p.Nk + 15) / 16;
  // fewest key splits the per-wave tile limit allows, then more while the
  // workgroups do not fill the chip (shorter chains per wave)
  int ksh = 0;
  while (ksh < 2 && (nt + (1 << ksh) - 1) >> ksh > S::NKT) ++ksh;
  if ((nt + (1 << ksh) - 1) >> ksh > S::NKT) return hipErrorInvalidValue;
  auto nwg_of = [&](int sh) { return (long long)p.BH * ((p.Nq + (16 << (2 - sh)) - 1) / (16 << (2 - sh))); };
  while (ksh < 2 && nt >= (2 << ksh) && nwg_of(ksh) < cus) ++ksh;
  const int tpw = (nt + (1 << ksh) - 1) >> ksh;  // tiles per wave
  switch (tpw) {
    case 1: return launch_short_k<TR, D, 1, kML>(p, ksh);
    case 2: return launch_short_k<TR, D, 2, kML>(p, ksh);
    case 3: return launch_short_k<TR, D, 3, kML>(p, ksh);
    case 4: return launch_short_k<TR, D, 4, kML>(p, ksh);
    default: break;
  }
  if constexpr (S::NKT >= 6) {
    if (tpw == 5) return launch_short_k<TR, D, 5, kML>(p, ksh);
    if (tpw == 6) return launch_short_k<TR, D, 6, kML>(p, ksh);
  }
  return hipErrorInvalidValue;
}

template <class TR, int D>
hipError_t launch_short_d(const Problem& p, int cus, bool shared) {
  if (shared) return p.ml ? launch_shared_t<TR, D, true>(p) : launch_shared_t<TR, D, false>(p);
  return p.ml ? launch_short_t<TR, D, true>(p, cus) : launch_short_t<TR, D, false>(p, cus);
}
template <class TR>
hipError_t launch_short_ty(const Problem& p, int cus, bool shared) {
  switch (p.d) {
    case 40: return launch_short_d<TR, 40>(p, cus, shared);
    case 80: return launch_short_d<TR, 80>(p, cus, shared);
    case 160: return launch_short_d<TR, 160>(p, cus, shared);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int short_max_keys(int d) {
  switch (d) {
    case 40: return ShortShape<40>::KEYS;
    case 80: return ShortShape<80>::KEYS;
    case 160: return ShortShape<160>::KEYS;
    default: return 0;
  }
}

// The two forms: shared where a head has at least one full workgroup's worth
// of 16-query groups (8) and at most 96 keys; per wave otherwise.  ATTN_SHORT=s /
// w forces the shared / per-wave form where the shape allows it.
hipError_t launch_short_flash(const Problem& p, int cus) {
  if (p.Nk < 1 || p.Nk > short_max_keys(p.d) || p.lay.H > 65535 || p.BH / p.lay.H > 65535) return hipErrorInvalidValue;
  const bool can_share = p.Nk <= 16 * kSharedTiles;
  bool shared = can_share && p.Nq >= 16 * kSharedW;
  const char* e = std::getenv("ATTN_SHORT");
  if (e && e[0] == 's') shared = can_share;
  if (e && e[0] == 'w') shared = false;
  return p.dt == ATTN_BF16 ? launch_short_ty<BF16>(p, cus, shared) : launch_short_ty<F16>(p, cus, shared);
}

}  // namespace attn
