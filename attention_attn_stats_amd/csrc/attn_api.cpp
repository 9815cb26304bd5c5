// C ABI of libattn.so: argument validation, dispatch to the kernels and the
// per-shape choice between the two attention forms.
//
// The choice mirrors "Speed Is All You Need" (Chen et al., news write-up,
// section on improving attention efficiency), where FlashAttention is used
// selectively -- for head dimension 40 on the GPUs studied, the partially
// fused softmax elsewhere -- because its kernel is register hungry.  Here the
// rule only seeds the default; ATTN_AUTO decides per shape by timing both
// forms on the device and caching the faster.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "attn.h"
#include "attn_internal.h"

namespace {

using attn::Problem;

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

attn_status check_common(int B, int H, int Nq, int Nk, int d, float scale, attn_dtype dt) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_INVALID_ARG;
  if (dt != ATTN_F32 && dt != ATTN_F16 && dt != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (d != 40 && d != 80 && d != 160) return ATTN_ERR_UNSUPPORTED;
  const long long bh = (long long)B * H;
  const long long lim = 0x7fffffffLL;
  if (bh > lim || bh * Nq > lim / 2 || bh * Nq * d > lim || bh * Nk * d > lim) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

Problem make(const void* q, const void* k, const void* v, void* out, float* ml, int B, int H, int Nq,
             int Nk, int d, float scale, attn_dtype dt, void* stream) {
  Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.ml = ml;
  p.a = nullptr;
  p.BH = B * H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.d = d;
  p.scale = scale;
  p.dt = dt;
  p.stream = (hipStream_t)stream;
  p.lay.q = attn::dense_strides(Nq, d, H);
  p.lay.o = p.lay.q;
  p.lay.k = attn::dense_strides(Nk, d, H);
  p.lay.v = p.lay.k;
  p.lay.H = H;
  return p;
}

attn_status to_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

attn_status run_stats(const Problem& p) {
  return to_status(p.dt == ATTN_F32 ? attn::launch_f32_stats(p) : attn::launch_mfma_stats(p));
}
attn_status run_pv(const Problem& p) {
  return to_status(p.dt == ATTN_F32 ? attn::launch_f32_pv(p) : attn::launch_mfma_pv(p));
}
attn_status run_flash(const Problem& p) {
  return to_status(p.dt == ATTN_F32 ? attn::launch_f32_flash(p) : attn::launch_mfma_flash(p));
}
attn_status run_pf(const Problem& p) {
  attn_status s = run_stats(p);
  return s == ATTN_OK ? run_pv(p) : s;
}

// Whether work on `st` is being captured into a graph (an error counts as
// yes: then nothing synchronises).
bool stream_capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return true;
  return cs != hipStreamCaptureStatusNone;
}

// Byte range [first, last] a [B][H][N][d] tensor of the problem spans.
struct Span {
  uintptr_t first, last;
};
Span span_of(const void* p, const attn::Strides& s, int B, int H, int N, int d, size_t esz) {
  const long long last = (long long)(B - 1) * s.batch + (long long)(H - 1) * s.head + (long long)(N - 1) * s.row + d;
  return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(last * (long long)esz) - 1};
}
bool overlap(const Span& a, const Span& b) { return a.first <= b.last && b.first <= a.last; }
// Whether out's memory range meets that of q, k or v (timing would then run
// a form over its own output).
bool out_meets_inputs(const Problem& p) {
  const size_t esz = p.dt == ATTN_F32 ? 4 : 2;
  const int B = p.BH / p.lay.H, H = p.lay.H;
  const Span o = span_of(p.out, p.lay.o, B, H, p.Nq, p.d, esz);
  return overlap(o, span_of(p.q, p.lay.q, B, H, p.Nq, p.d, esz)) ||
         overlap(o, span_of(p.k, p.lay.k, B, H, p.Nk, p.d, esz)) ||
         overlap(o, span_of(p.v, p.lay.v, B, H, p.Nk, p.d, esz));
}

// ---- variant cache -------------------------------------------------------
typedef std::tuple<int, int, int, int, int, int> Key;  // BH, Nq, Nk, d, dtype, device
std::mutex g_mu;
std::map<Key, attn_variant> g_cache;

attn_variant env_override() {
  const char* e = std::getenv("ATTN_VARIANT");
  if (!e) return ATTN_AUTO;
  if (!std::strcmp(e, "pf") || !std::strcmp(e, "partial_fused")) return ATTN_PARTIAL_FUSED;
  if (!std::strcmp(e, "flash")) return ATTN_FLASH;
  return ATTN_AUTO;
}

int select_iters() {
  const char* e = std::getenv("ATTN_SELECT_ITERS");
  const int n = e ? std::atoi(e) : 5;
  return std::min(std::max(n, 1), 100);
}

Key key_of(const Problem& p) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  return Key(p.BH, p.Nq, p.Nk, p.d, (int)p.dt, dev);
}

// Median time (ms) of `iters` runs of one variant, after one warm-up run.
attn_status time_variant(const Problem& p, attn_variant var, int iters, float* ms_out) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return ATTN_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return ATTN_ERR_HIP;
  }
  Problem pf = p;
  pf.ml = nullptr;  // the single pass runs without the statistics output, as attn_forward issues it
  auto run = [&]() { return var == ATTN_FLASH ? run_flash(pf) : run_pf(p); };
  attn_status st = run();
  float times[100];
  for (int i = 0; i < iters && st == ATTN_OK; ++i) {
    if (hipEventRecord(e0, p.stream) != hipSuccess) st = ATTN_ERR_HIP;
    if (st == ATTN_OK) st = run();
    if (st == ATTN_OK && hipEventRecord(e1, p.stream) != hipSuccess) st = ATTN_ERR_HIP;
    if (st == ATTN_OK && hipEventSynchronize(e1) != hipSuccess) st = ATTN_ERR_HIP;
    if (st == ATTN_OK && hipEventElapsedTime(&times[i], e0, e1) != hipSuccess) st = ATTN_ERR_HIP;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != ATTN_OK) return st;
  std::sort(times, times + iters);
  *ms_out = times[iters / 2];
  return ATTN_OK;
}

// Times both variants on the problem's buffers and returns the faster; the
// last run is the winner's, so the outputs are those of the chosen variant.
attn_status measure(const Problem& p, attn_variant* out) {
  const int iters = select_iters();
  float t_pf = 0.f, t_fl = 0.f;
  attn_status st = time_variant(p, ATTN_PARTIAL_FUSED, iters, &t_pf);
  if (st == ATTN_OK) st = time_variant(p, ATTN_FLASH, iters, &t_fl);
  if (st != ATTN_OK) return st;
  *out = t_fl <= t_pf ? ATTN_FLASH : ATTN_PARTIAL_FUSED;
  if (*out == ATTN_PARTIAL_FUSED) st = run_pf(p);  // FLASH already ran last
  return st;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension, element type or variant";
    case ATTN_ERR_HIP: return "HIP runtime error";
    default: break;
  }
  return "unknown status";
}

attn_variant attn_default_variant(int d) { return d == 40 ? ATTN_FLASH : ATTN_PARTIAL_FUSED; }

attn_status attn_stats(const void* q, const void* k, float* ml, int B, int H, int Nq, int Nk, int d,
                       float scale, attn_dtype dt, void* stream) {
  if (!q || !k || !ml || !aligned16(q) || !aligned16(k) || ((uintptr_t)ml & 7u)) return ATTN_ERR_INVALID_ARG;
  attn_status s = check_common(B, H, Nq, Nk, d, scale, dt);
  if (s != ATTN_OK) return s;
  return run_stats(make(q, k, nullptr, nullptr, ml, B, H, Nq, Nk, d, scale, dt, stream));
}

attn_status attn_pv(const void* q, const void* k, const void* v, const float* ml, void* out, int B, int H,
                    int Nq, int Nk, int d, float scale, attn_dtype dt, void* stream) {
  if (!q || !k || !v || !ml || !out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)ml & 7u))
    return ATTN_ERR_INVALID_ARG;
  attn_status s = check_common(B, H, Nq, Nk, d, scale, dt);
  if (s != ATTN_OK) return s;
  return run_pv(make(q, k, v, out, const_cast<float*>(ml), B, H, Nq, Nk, d, scale, dt, stream));
}

attn_status attn_flash(const void* q, const void* k, const void* v, void* out, float* ml_out, int B, int H,
                       int Nq, int Nk, int d, float scale, attn_dtype dt, void* stream) {
  if (!q || !k || !v || !out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)ml_out & 7u))
    return ATTN_ERR_INVALID_ARG;
  attn_status s = check_common(B, H, Nq, Nk, d, scale, dt);
  if (s != ATTN_OK) return s;
  return run_flash(make(q, k, v, out, ml_out, B, H, Nq, Nk, d, scale, dt, stream));
}

// ---- strided tensors ------------------------------------------------------
namespace {
// A strided [B][H][N][d] tensor: non-negative strides, rows of at least d
// and at most 2^20 elements, every row 16-byte aligned (strides in multiples
// of 16 bytes), the whole tensor within 2^31 elements and one head's rows
// within 2^30 (the kernels address a head's rows, and a block of 64 rows,
// with 32-bit byte offsets).
attn_status check_strides(const attn_strides& s, int B, int H, int N, int d, attn_dtype dt) {
  const long long unit = dt == ATTN_F32 ? 4 : 8;  // elements per 16 bytes
  if (s.batch < 0 || s.head < 0 || s.row < d || s.row > (1LL << 20)) return ATTN_ERR_INVALID_ARG;
  if (s.batch % unit || s.head % unit || s.row % unit) return ATTN_ERR_INVALID_ARG;
  const long long head_extent = (long long)(N - 1) * s.row + d;
  if (head_extent >= (1LL << 30)) return ATTN_ERR_INVALID_ARG;
  if ((long long)(B - 1) * s.batch + (long long)(H - 1) * s.head + head_extent >= 0x7fffffffLL)
    return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}
attn::Strides to_internal(const attn_strides& s) {
  attn::Strides r;
  r.batch = s.batch;
  r.head = s.head;
  r.row = (int)s.row;
  return r;
}
// Validates the layout of the tensors an operation uses (v, out optional) and
// installs it in p.
attn_status apply_layout(Problem& p, const attn_layout* lay, int B, int H, bool has_v, bool has_out) {
  if (!lay) return ATTN_OK;  // dense
  attn_status s = check_strides(lay->q, B, H, p.Nq, p.d, p.dt);
  if (s == ATTN_OK) s = check_strides(lay->k, B, H, p.Nk, p.d, p.dt);
  if (s == ATTN_OK && has_v) s = check_strides(lay->v, B, H, p.Nk, p.d, p.dt);
  if (s == ATTN_OK && has_out) s = check_strides(lay->out, B, H, p.Nq, p.d, p.dt);
  if (s != ATTN_OK) return s;
  p.lay.q = to_internal(lay->q);
  p.lay.k = to_internal(lay->k);
  if (has_v) p.lay.v = to_internal(lay->v);
  if (has_out) p.lay.o = to_internal(lay->out);
  return ATTN_OK;
}
}  // namespace

attn_status attn_forward_strided(const void* q, const void* k, const void* v, void* out, float* ml,
                                 const attn_layout* lay, int B, int H, int Nq, int Nk, int d, float scale,
                                 attn_variant var, attn_dtype dt, void* stream) {
  if (!q || !k || !v || !out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)ml & 7u))
    return ATTN_ERR_INVALID_ARG;
  if (var != ATTN_AUTO && var != ATTN_PARTIAL_FUSED && var != ATTN_FLASH) return ATTN_ERR_UNSUPPORTED;
  attn_status s = check_common(B, H, Nq, Nk, d, scale, dt);
  if (s != ATTN_OK) return s;
  if (var == ATTN_PARTIAL_FUSED && !ml) return ATTN_ERR_INVALID_ARG;
  Problem p = make(q, k, v, out, ml, B, H, Nq, Nk, d, scale, dt, stream);
  s = apply_layout(p, lay, B, H, true, true);
  if (s != ATTN_OK) return s;
  if (var == ATTN_AUTO) {
    const attn_variant forced = env_override();
    if (forced != ATTN_AUTO) var = forced;
    if (var == ATTN_PARTIAL_FUSED && !ml) var = ATTN_FLASH;
  }
  if (var == ATTN_AUTO) {
    if (!ml) return run_flash(p);
    const Key key = key_of(p);
    {
      std::lock_guard<std::mutex> g(g_mu);
      auto it = g_cache.find(key);
      if (it != g_cache.end()) var = it->second;
    }
    if (var == ATTN_AUTO && (stream_capturing(p.stream) || out_meets_inputs(p))) {
      // timing synchronises, which a stream being captured into a graph
      // must not do, and runs both forms several times, which an output
      // sharing memory with an input would corrupt: the rule-of-thumb
      // choice, not cached
      var = attn_default_variant(p.d);
    }
    if (var == ATTN_AUTO) {
      attn_variant chosen = ATTN_AUTO;
      s = measure(p, &chosen);
      if (s != ATTN_OK) return s;
      std::lock_guard<std::mutex> g(g_mu);
      g_cache[key] = chosen;
      return ATTN_OK;  // measure() left the chosen variant's outputs in place
    }
  }
  if (var == ATTN_FLASH) {
    Problem pf = p;
    pf.ml = nullptr;  // the single pass needs no statistics buffer
    return run_flash(pf);
  }
  return run_pf(p);
}

attn_status attn_forward(const void* q, const void* k, const void* v, void* out, float* ml, int B, int H,
                         int Nq, int Nk, int d, float scale, attn_variant var, attn_dtype dt, void* stream) {
  return attn_forward_strided(q, k, v, out, ml, nullptr, B, H, Nq, Nk, d, scale, var, dt, stream);
}

// ---- the partially fused form over a stored logit matrix ------------------
namespace {
// A = [B][H][Nq][Nk] float32: a head's part must stay below 2^31 bytes (the
// kernels address it with 32-bit offsets), the whole within size_t.
attn_status check_scores(int B, int H, int Nq, int Nk) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_INVALID_ARG;
  if ((long long)Nq * Nk * 4 >= 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
  if ((long long)B * H * Nq >= 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}
}  // namespace

attn_status attn_scores(const void* q, const void* k, float* a, int B, int H, int Nq, int Nk, int d,
                        float scale, attn_dtype dt, void* stream) {
  if (!q || !k || !a || !aligned16(q) || !aligned16(k) || ((uintptr_t)a & 3u)) return ATTN_ERR_INVALID_ARG;
  attn_status s = check_common(B, H, Nq, Nk, d, scale, dt);
  if (s == ATTN_OK) s = check_scores(B, H, Nq, Nk);
  if (s != ATTN_OK) return s;
  if (dt == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  return to_status(attn::launch_scores(make(q, k, nullptr, nullptr, nullptr, B, H, Nq, Nk, d, scale, dt, stream), a));
}

attn_status attn_scores_stats(const float* a, float* ml, int B, int H, int Nq, int Nk, void* stream) {
  if (!a || !ml || ((uintptr_t)a & 3u) || ((uintptr_t)ml & 7u)) return ATTN_ERR_INVALID_ARG;
  attn_status s = check_scores(B, H, Nq, Nk);
  if (s != ATTN_OK) return s;
  return to_status(attn::launch_scores_stats(a, ml, (long long)B * H * Nq, Nk, (hipStream_t)stream));
}

attn_status attn_scores_pv(const float* a, const float* ml, const void* v, void* out, int B, int H, int Nq,
                           int Nk, int d, attn_dtype dt, void* stream) {
  if (!a || !ml || !v || !out || ((uintptr_t)a & 3u) || ((uintptr_t)ml & 7u) || !aligned16(v) || !aligned16(out))
    return ATTN_ERR_INVALID_ARG;
  attn_status s = check_common(B, H, Nq, Nk, d, 1.f, dt);
  if (s == ATTN_OK) s = check_scores(B, H, Nq, Nk);
  if (s != ATTN_OK) return s;
  if (dt == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  Problem p = make(nullptr, nullptr, v, out, const_cast<float*>(ml), B, H, Nq, Nk, d, 1.f, dt, stream);
  p.a = a;
  return to_status(attn::launch_mfma_pv_scores(p));
}


attn_status attn_stats_strided(const void* q, const void* k, float* ml, const attn_layout* lay, int B, int H,
                               int Nq, int Nk, int d, float scale, attn_dtype dt, void* stream) {
  if (!q || !k || !ml || !aligned16(q) || !aligned16(k) || ((uintptr_t)ml & 7u)) return ATTN_ERR_INVALID_ARG;
  attn_status s = check_common(B, H, Nq, Nk, d, scale, dt);
  if (s != ATTN_OK) return s;
  Problem p = make(q, k, nullptr, nullptr, ml, B, H, Nq, Nk, d, scale, dt, stream);
  s = apply_layout(p, lay, B, H, false, false);
  return s != ATTN_OK ? s : run_stats(p);
}

attn_status attn_pv_strided(const void* q, const void* k, const void* v, const float* ml, void* out,
                            const attn_layout* lay, int B, int H, int Nq, int Nk, int d, float scale,
                            attn_dtype dt, void* stream) {
  if (!q || !k || !v || !ml || !out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)ml & 7u))
    return ATTN_ERR_INVALID_ARG;
  attn_status s = check_common(B, H, Nq, Nk, d, scale, dt);
  if (s != ATTN_OK) return s;
  Problem p = make(q, k, v, out, const_cast<float*>(ml), B, H, Nq, Nk, d, scale, dt, stream);
  s = apply_layout(p, lay, B, H, true, true);
  return s != ATTN_OK ? s : run_pv(p);
}

attn_status attn_flash_strided(const void* q, const void* k, const void* v, void* out, float* ml_out,
                               const attn_layout* lay, int B, int H, int Nq, int Nk, int d, float scale,
                               attn_dtype dt, void* stream) {
  if (!q || !k || !v || !out) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || ((uintptr_t)ml_out & 7u))
    return ATTN_ERR_INVALID_ARG;
  attn_status s = check_common(B, H, Nq, Nk, d, scale, dt);
  if (s != ATTN_OK) return s;
  Problem p = make(q, k, v, out, ml_out, B, H, Nq, Nk, d, scale, dt, stream);
  s = apply_layout(p, lay, B, H, true, true);
  return s != ATTN_OK ? s : run_flash(p);
}

// ---- group normalisation and the GELU-gated product ----------------------
namespace {
size_t elem_size(attn_dtype dt) { return dt == ATTN_F32 ? 4 : 2; }
bool aligned_to(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }
}  // namespace

namespace {
// Validates a group-normalisation problem and fills p (all but the workspace).
attn_status gn_problem(const void* x, const void* gamma, const void* beta, void* y, int N, int C, int HW, int G,
                       float eps, attn_dtype dt, void* stream, attn::GroupNormProblem* p) {
  if (dt != ATTN_F32 && dt != ATTN_F16 && dt != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!x || !y) return ATTN_ERR_INVALID_ARG;
  if (N < 1 || C < 1 || HW < 1 || G < 1 || C % G != 0) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return ATTN_ERR_INVALID_ARG;
  if ((long long)N * C * HW >= (1LL << 40) || (long long)(C / G) * HW >= 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
  const size_t es = elem_size(dt);
  if (!aligned_to(x, es) || !aligned_to(y, es) || (gamma && !aligned_to(gamma, es)) ||
      (beta && !aligned_to(beta, es)))
    return ATTN_ERR_INVALID_ARG;
  p->x = x;
  p->gamma = gamma;
  p->beta = beta;
  p->y = y;
  p->workspace = nullptr;
  p->workspace_bytes = 0;
  p->N = N;
  p->C = C;
  p->HW = HW;
  p->G = G;
  p->eps = eps;
  p->dt = dt;
  p->stream = (hipStream_t)stream;
  return ATTN_OK;
}
}  // namespace

attn_status attn_group_norm(const void* x, const void* gamma, const void* beta, void* y, void* workspace,
                            size_t workspace_bytes, int N, int C, int HW, int G, float eps, attn_dtype dt,
                            void* stream) {
  attn::GroupNormProblem p;
  attn_status s = gn_problem(x, gamma, beta, y, N, C, HW, G, eps, dt, stream, &p);
  if (s != ATTN_OK) return s;
  if (workspace && !aligned_to(workspace, 8)) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::group_norm_workspace(p);
  if (need && (!workspace || workspace_bytes < need)) return ATTN_ERR_INVALID_ARG;
  p.workspace = workspace;
  p.workspace_bytes = workspace ? workspace_bytes : 0;
  return to_status(attn::launch_group_norm(p));
}

attn_status attn_group_norm_static(const void* x, const void* gamma, const void* beta, void* y, int N, int C,
                                   int HW, int G, float eps, attn_dtype dt, void* stream) {
  attn::GroupNormProblem p;
  attn_status s = gn_problem(x, gamma, beta, y, N, C, HW, G, eps, dt, stream, &p);
  if (s != ATTN_OK) return s;
  const size_t need = attn::group_norm_workspace(p);
  if (need > attn::kGnStaticScratchBytes) return ATTN_ERR_INVALID_ARG;
  if (need) {
    void* ws = nullptr;
    if (attn::group_norm_static_scratch(&ws) != hipSuccess) return ATTN_ERR_HIP;
    p.workspace = ws;
    p.workspace_bytes = attn::kGnStaticScratchBytes;
  }
  return to_status(attn::launch_group_norm(p));
}

size_t attn_group_norm_workspace_size(const void* x, const void* y, int N, int C, int HW, int G,
                                      attn_dtype dt) {
  attn::GroupNormProblem p;
  if (gn_problem(x, nullptr, nullptr, const_cast<void*>(y), N, C, HW, G, 0.f, dt, nullptr, &p) != ATTN_OK) return 0;
  return attn::group_norm_workspace(p);
}

attn_status attn_geglu(const void* h, void* out, int rows, int F, attn_dtype dt, void* stream) {
  if (dt != ATTN_F32 && dt != ATTN_F16 && dt != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!h || !out || rows < 1 || F < 1) return ATTN_ERR_INVALID_ARG;
  if ((long long)rows * F >= (1LL << 31) - 512) return ATTN_ERR_INVALID_ARG;
  const size_t es = elem_size(dt);
  if (!aligned_to(h, es) || !aligned_to(out, es)) return ATTN_ERR_INVALID_ARG;
  attn::GegluProblem p;
  p.h = h;
  p.out = out;
  p.rows = rows;
  p.F = F;
  p.dt = dt;
  p.stream = (hipStream_t)stream;
  return to_status(attn::launch_geglu(p));
}

attn_variant attn_select(int B, int H, int Nq, int Nk, int d, attn_dtype dt, void* stream) {
  if (check_common(B, H, Nq, Nk, d, 1.f, dt) != ATTN_OK) return ATTN_AUTO;
  const attn_variant forced = env_override();
  if (forced != ATTN_AUTO) return forced;
  Problem p = make(nullptr, nullptr, nullptr, nullptr, nullptr, B, H, Nq, Nk, d, 1.f / std::sqrt((float)d),
                   dt, stream);
  const Key key = key_of(p);
  {
    std::lock_guard<std::mutex> g(g_mu);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) return it->second;
  }
  // timing allocates and synchronises: not on a stream being captured
  if (stream_capturing(p.stream)) return attn_default_variant(d);
  const size_t esz = dt == ATTN_F32 ? 4 : 2;
  const size_t nq = (size_t)p.BH * Nq * d * esz, nk = (size_t)p.BH * Nk * d * esz;
  void *bq = nullptr, *bk = nullptr, *bv = nullptr, *bo = nullptr, *bml = nullptr;
  attn_variant chosen = ATTN_AUTO;
  if (hipMalloc(&bq, nq) == hipSuccess && hipMalloc(&bk, nk) == hipSuccess && hipMalloc(&bv, nk) == hipSuccess &&
      hipMalloc(&bo, nq) == hipSuccess && hipMalloc(&bml, (size_t)p.BH * Nq * 2 * sizeof(float)) == hipSuccess &&
      attn::launch_fill_uniform(bq, nq / esz, dt, 1, p.stream) == hipSuccess &&
      attn::launch_fill_uniform(bk, nk / esz, dt, 2, p.stream) == hipSuccess &&
      attn::launch_fill_uniform(bv, nk / esz, dt, 3, p.stream) == hipSuccess) {
    p.q = bq;
    p.k = bk;
    p.v = bv;
    p.out = bo;
    p.ml = (float*)bml;
    if (measure(p, &chosen) != ATTN_OK) chosen = ATTN_AUTO;
    (void)hipStreamSynchronize(p.stream);
  }
  (void)hipFree(bq);
  (void)hipFree(bk);
  (void)hipFree(bv);
  (void)hipFree(bo);
  (void)hipFree(bml);
  if (chosen != ATTN_AUTO) {
    std::lock_guard<std::mutex> g(g_mu);
    g_cache[key] = chosen;
  }
  return chosen;
}

void attn_select_reset(void) {
  std::lock_guard<std::mutex> g(g_mu);
  g_cache.clear();
}

}  // extern "C"
