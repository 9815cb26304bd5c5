// Seeded stand-in inputs for timing a shape without the caller's data (the
// per-shape variant selector, attn_select): element i takes a value uniform
// on [-sqrt 3, sqrt 3) (zero mean, unit variance, the spread of normalised
// activations), from a counter-based hash of (seed, i): SplitMix64's output
// function (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014) on seed * 2^32 + i.  Timing only: no result of
// the library depends on these values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// mode 0: float32, 1: fp16, 2: bf16 (round to nearest even)
__global__ void fill_uniform_kernel(void* p, size_t n, uint64_t seed, int mode) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint64_t h = mix64((seed << 32) + i);
    const float u = (float)(h >> 40) * (1.0f / 16777216.0f);      // [0, 1), 24 bits
    const float x = (2.0f * u - 1.0f) * 1.7320508f;
    if (mode == 0) {
      ((float*)p)[i] = x;
    } else if (mode == 1) {
      ((_Float16*)p)[i] = (_Float16)x;
    } else {
      const uint32_t b = __float_as_uint(x);
      ((uint16_t*)p)[i] = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
    }
  }
}

}  // namespace

hipError_t launch_fill_uniform(void* p, size_t n, attn_dtype dt, unsigned seed, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int mode = dt == ATTN_F32 ? 0 : dt == ATTN_F16 ? 1 : 2;
  const size_t want = (n + 255) / 256;
  const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(fill_uniform_kernel, dim3(grid), dim3(256), 0, stream, p, n, (uint64_t)seed, mode);
  return hipGetLastError();
}

}  // namespace attn
