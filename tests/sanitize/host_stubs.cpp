// Stand-ins for the kernel launchers, so that the C ABI's host code
// (attn_api.cpp: argument validation, stride and layout arithmetic, the
// variant cache) can be built and run on a machine without a GPU under
// AddressSanitizer / UndefinedBehaviorSanitizer.  Every launcher records
// that it was reached and returns success without touching the pointers.
#include <cstddef>

#include "attn_internal.h"

namespace attn {
int g_launches = 0;
hipError_t launch_mfma_stats(const Problem&) { ++g_launches; return hipSuccess; }
hipError_t launch_mfma_pv(const Problem&) { ++g_launches; return hipSuccess; }
hipError_t launch_mfma_flash(const Problem&) { ++g_launches; return hipSuccess; }
hipError_t launch_fa40_flash(const Problem&, int) { ++g_launches; return hipSuccess; }
hipError_t launch_fa40_pv(const Problem&, int) { ++g_launches; return hipSuccess; }
hipError_t launch_scores(const Problem&, float*) { ++g_launches; return hipSuccess; }
hipError_t launch_scores_stats(const float*, float*, long long, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_mfma_pv_scores(const Problem&) { ++g_launches; return hipSuccess; }
hipError_t launch_fill_uniform(void*, size_t, attn_dtype, unsigned, hipStream_t) { ++g_launches; return hipSuccess; }
// a plan-like size: 16 bytes per (group, slice) for groups too large for one workgroup
size_t group_norm_workspace(const GroupNormProblem& p) {
  const long long group = (long long)(p.C / p.G) * p.HW;
  return group > 131072 ? (size_t)p.N * p.G * ((group + 131071) / 131072) * 16 : 0;
}
hipError_t launch_group_norm(const GroupNormProblem&) { ++g_launches; return hipSuccess; }
static unsigned long long fake_scratch[kGnStaticScratchBytes / 8];
hipError_t group_norm_static_scratch(void** ptr) { *ptr = fake_scratch; return hipSuccess; }
hipError_t launch_geglu(const GegluProblem&) { ++g_launches; return hipSuccess; }
hipError_t launch_f32_stats(const Problem&) { ++g_launches; return hipSuccess; }
hipError_t launch_f32_pv(const Problem&) { ++g_launches; return hipSuccess; }
hipError_t launch_f32_flash(const Problem&) { ++g_launches; return hipSuccess; }
}  // namespace attn
