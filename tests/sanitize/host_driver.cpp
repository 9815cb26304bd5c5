// Calls every entry point of include/attn.h with invalid arguments (which
// must be refused before anything is launched) and with valid ones on fake
// device pointers (reaching the stand-in launchers of host_stubs.cpp), so
// that an AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI's
// host code reports any out-of-bounds access or undefined arithmetic in the
// validation, stride, overflow and layout checks.  Exit status 0 when every
// return code is the documented one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "attn.h"

namespace attn {
extern int g_launches;
}

static int failures = 0;
#define EXPECT(expr, want)                                                                \
  do {                                                                                    \
    const int got_ = (int)(expr);                                                         \
    if (got_ != (int)(want)) {                                                            \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_, \
                   (int)(want));                                                          \
      ++failures;                                                                         \
    }                                                                                     \
  } while (0)

int main() {
  // fake device pointers, 256-byte aligned, never dereferenced
  void* P = (void*)(uintptr_t)0x10000000;
  void* Q = (void*)(uintptr_t)0x20000000;
  float* ML = (float*)(uintptr_t)0x30000000;
  const attn_dtype H16 = ATTN_F16;
  const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();
  // ---- attn_stats / attn_pv / attn_flash / attn_forward: refusals
  for (int d : {40, 80, 160}) {
    EXPECT(attn_stats(nullptr, P, ML, 1, 1, 16, 16, d, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_stats(P, P, ML, 0, 1, 16, 16, d, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_stats(P, P, ML, 1, 1, 0, 16, d, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_stats(P, P, ML, 1, 1, 16, 0, d, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_stats(P, P, ML, 1, 1, 16, 16, d, 0.f, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_stats(P, P, ML, 1, 1, 16, 16, d, nan, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_stats(P, P, ML, 1, 1, 16, 16, d, inf, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_stats((char*)P + 2, P, ML, 1, 1, 16, 16, d, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_pv(P, P, P, nullptr, Q, 1, 1, 16, 16, d, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_flash(P, P, P, nullptr, nullptr, 1, 1, 16, 16, d, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);
    EXPECT(attn_forward(P, P, P, Q, ML, 1, 1, 16, 16, d, 0.1f, (attn_variant)7, H16, nullptr),
           ATTN_ERR_UNSUPPORTED);
    EXPECT(attn_forward(P, P, P, Q, nullptr, 1, 1, 16, 16, d, 0.1f, ATTN_PARTIAL_FUSED, H16, nullptr),
           ATTN_ERR_INVALID_ARG);
  }
  EXPECT(attn_stats(P, P, ML, 1, 1, 16, 16, 64, 0.1f, H16, nullptr), ATTN_ERR_UNSUPPORTED);
  EXPECT(attn_stats(P, P, ML, 1, 1, 16, 16, 40, 0.1f, (attn_dtype)9, nullptr), ATTN_ERR_UNSUPPORTED);
  // sizes whose products overflow 32 bits must be refused, not wrapped
  EXPECT(attn_stats(P, P, ML, 1 << 20, 1 << 12, 1 << 12, 16, 40, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);
  EXPECT(attn_flash(P, P, P, Q, nullptr, 1, 1, 0x7fffffff, 16, 160, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);
  // ---- valid calls reach a launcher
  int before = attn::g_launches;
  EXPECT(attn_stats(P, P, ML, 2, 8, 4096, 4096, 40, 0.158f, H16, nullptr), ATTN_OK);
  EXPECT(attn_pv(P, P, P, ML, Q, 2, 8, 4096, 4096, 40, 0.158f, H16, nullptr), ATTN_OK);
  EXPECT(attn_flash(P, P, P, Q, ML, 1, 1, 77, 3, 80, 0.1f, ATTN_BF16, nullptr), ATTN_OK);
  EXPECT(attn_flash(P, P, P, Q, nullptr, 1, 3, 1, 1, 160, 0.1f, ATTN_F32, nullptr), ATTN_OK);
  EXPECT(attn_forward(P, P, P, Q, ML, 1, 1, 64, 64, 40, 0.1f, ATTN_FLASH, H16, nullptr), ATTN_OK);
  EXPECT(attn_forward(P, P, P, Q, ML, 1, 1, 64, 64, 40, 0.1f, ATTN_PARTIAL_FUSED, H16, nullptr), ATTN_OK);
  if (attn::g_launches <= before) {
    std::fprintf(stderr, "valid calls reached no launcher\n");
    ++failures;
  }
  // ---- strided forms: layout checks
  attn_layout lay{};
  const int B = 2, H = 8, N = 1024, d = 40;
  lay.q = attn_strides{(long long)N * H * d, d, H * d};  // [B, N, H*d] viewed as [B, H, N, d]
  lay.k = lay.q;
  lay.v = lay.q;
  lay.out = lay.q;
  EXPECT(attn_flash_strided(P, P, P, Q, nullptr, &lay, B, H, N, N, d, 0.158f, H16, nullptr), ATTN_OK);
  EXPECT(attn_forward_strided(P, P, P, Q, ML, &lay, B, H, N, N, d, 0.158f, ATTN_FLASH, H16, nullptr), ATTN_OK);
  EXPECT(attn_stats_strided(P, P, ML, &lay, B, H, N, N, d, 0.158f, H16, nullptr), ATTN_OK);
  EXPECT(attn_pv_strided(P, P, P, ML, Q, &lay, B, H, N, N, d, 0.158f, H16, nullptr), ATTN_OK);
  attn_layout bad = lay;
  bad.q.row = d - 1;  // a row shorter than d
  EXPECT(attn_flash_strided(P, P, P, Q, nullptr, &bad, B, H, N, N, d, 0.158f, H16, nullptr), ATTN_ERR_INVALID_ARG);
  bad = lay;
  bad.k.head = -8;  // negative stride
  EXPECT(attn_flash_strided(P, P, P, Q, nullptr, &bad, B, H, N, N, d, 0.158f, H16, nullptr), ATTN_ERR_INVALID_ARG);
  bad = lay;
  bad.v.row = H * d + 1;  // not a multiple of 16 bytes
  EXPECT(attn_flash_strided(P, P, P, Q, nullptr, &bad, B, H, N, N, d, 0.158f, H16, nullptr), ATTN_ERR_INVALID_ARG);
  bad = lay;
  bad.q.batch = (long long)1 << 40;  // the whole tensor beyond 2^31 elements
  EXPECT(attn_flash_strided(P, P, P, Q, nullptr, &bad, B, H, N, N, d, 0.158f, H16, nullptr), ATTN_ERR_INVALID_ARG);
  bad = lay;
  bad.out = attn_strides{0, 0, 0};  // every output row on the same memory
  EXPECT(attn_flash_strided(P, P, P, Q, nullptr, &bad, B, H, N, N, d, 0.158f, H16, nullptr), ATTN_ERR_INVALID_ARG);
  EXPECT(attn_flash_strided(P, P, P, Q, nullptr, nullptr, B, H, N, N, d, 0.158f, H16, nullptr), ATTN_OK);
  // ---- the stored-logit form
  EXPECT(attn_scores(P, P, ML, 1, 1, 46341, 46341, 40, 0.1f, H16, nullptr), ATTN_ERR_INVALID_ARG);  // head > 2^31 B
  EXPECT(attn_scores(P, P, ML, 2, 8, 1024, 1024, 40, 0.1f, H16, nullptr), ATTN_OK);
  EXPECT(attn_scores_stats(ML, ML, 2, 8, 1024, 1024, nullptr), ATTN_OK);
  EXPECT(attn_scores_stats(nullptr, ML, 2, 8, 1024, 1024, nullptr), ATTN_ERR_INVALID_ARG);
  EXPECT(attn_scores_pv(ML, ML, P, Q, 2, 8, 1024, 1024, 40, H16, nullptr), ATTN_OK);
  EXPECT(attn_scores_pv(ML, ML, P, Q, 0, 8, 1024, 1024, 40, H16, nullptr), ATTN_ERR_INVALID_ARG);
  // ---- group normalisation and the gated product
  EXPECT(attn_group_norm(P, nullptr, nullptr, Q, nullptr, 0, 2, 320, 4096, 32, 1e-5f, H16, nullptr), ATTN_OK);
  EXPECT(attn_group_norm(P, nullptr, nullptr, Q, nullptr, 0, 1, 128, 65536, 32, 1e-5f, H16, nullptr),
         ATTN_ERR_INVALID_ARG);  // needs a workspace
  EXPECT(attn_group_norm(P, nullptr, nullptr, Q, ML, 1 << 20, 1, 128, 65536, 32, 1e-5f, H16, nullptr), ATTN_OK);
  EXPECT(attn_group_norm(P, nullptr, nullptr, Q, nullptr, 0, 2, 30, 64, 4, 1e-5f, H16, nullptr), ATTN_ERR_INVALID_ARG);
  EXPECT(attn_group_norm(P, nullptr, nullptr, Q, nullptr, 0, 2, 32, 64, 32, -1.f, H16, nullptr), ATTN_ERR_INVALID_ARG);
  EXPECT(attn_group_norm_static(P, nullptr, nullptr, Q, 1, 128, 65536, 32, 1e-5f, H16, nullptr), ATTN_OK);
  EXPECT(attn_group_norm_static(P, nullptr, nullptr, Q, 4096, 128, 65536, 32, 1e-5f, H16, nullptr),
         ATTN_ERR_INVALID_ARG);  // beyond the fixed scratch
  EXPECT(attn_group_norm_workspace_size(P, Q, 2, 30, 64, 4, H16), 0);
  EXPECT(attn_geglu(P, Q, 8192, 1280, H16, nullptr), ATTN_OK);
  EXPECT(attn_geglu(P, Q, 1 << 16, 1 << 15, H16, nullptr), ATTN_ERR_INVALID_ARG);
  EXPECT(attn_geglu(nullptr, Q, 4, 8, H16, nullptr), ATTN_ERR_INVALID_ARG);
  // ---- selection (no device here: timing fails and nothing is cached)
  EXPECT(attn_default_variant(40), ATTN_FLASH);
  EXPECT(attn_default_variant(80), ATTN_PARTIAL_FUSED);
  EXPECT(attn_select(0, 1, 16, 16, 40, H16, nullptr), ATTN_AUTO);
  attn_select_reset();
  for (int s = 0; s < 6; ++s)
    if (!attn_status_string((attn_status)s)) ++failures;
  std::printf(failures ? "FAIL %d\n" : "OK\n", failures);
  return failures ? 1 : 0;
}
