// probe.hip -- measurement helper: the ceiling of the MFMA form the NVFP4
// GEMM issues (v_mfma_f32_32x32x16_f16) on operands with the values the GEMM
// feeds it (decoded E2M1 codes times E4M3 block scales), without memory
// traffic.  One wave per SIMD and sixteen 32x32 accumulators per wave, as in
// the GEMM; the operands change every K step.  Not part of the method: the
// benchmark reports its rate beside the published peak.
#include "nvfp4.h"
#include "nvfp4_device.h"

namespace nvfp4 {
namespace {

constexpr int kProbeBlocks = 1024, kProbeThreads = 256;

__global__ void __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_probe_mfma(int64_t iters, float *out) {
  float16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  // two operand sets of E2M1 values times E4M3 mantissas (1 + m/8) times a
  // power of two, from a per-lane linear congruential sequence
  half8_t a[2][4], b[2][4];
  const float q[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  uint32_t st = (uint32_t)(blockIdx.x * kProbeThreads + threadIdx.x) * 2654435761u + 12345u;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        st = st * 1664525u + 1013904223u;
        a[s][f][e] = (_Float16)(((st >> 9) & 1 ? -1.0f : 1.0f) * q[(st >> 12) & 7] * (1.0f + ((st >> 20) & 7) / 8.0f) * 4.0f);
        st = st * 1664525u + 1013904223u;
        b[s][f][e] = (_Float16)(((st >> 9) & 1 ? -1.0f : 1.0f) * q[(st >> 12) & 7] * (1.0f + ((st >> 20) & 7) / 8.0f) * 4.0f);
      }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int jj = (i & 1) ? 3 - j : j;
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s][i], b[s][jj], acc[i][jj], 0, 0, 0);
        }
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) t += acc[i][j][e];
  out[blockIdx.x * kProbeThreads + threadIdx.x] = t;
}

// The random bits of stochastic rounding alone: Philox4x32-10 (the same
// device routine the encodes use) for counters 0 .. calls-1, one call per 8
// elements, XOR-folded so the work stays live; no memory traffic besides one
// word per thread.  Its time is the floor the RNG contract puts under every
// stochastic-rounding encode of 8 * calls elements.
__global__ void __launch_bounds__(kProbeThreads) k_probe_philox(int64_t calls, uint64_t seed, uint32_t *out) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < calls; i += stride) {
    const uint4 w = sr_words8((uint64_t)i, seed, 0);
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  out[blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace
}  // namespace nvfp4

extern "C" int nvfp4_probe_philox(int64_t calls, uint32_t *out, void *hip_stream) {
  if (!out) return NVFP4_ERR_NULL;
  if (calls < 0) return NVFP4_ERR_SHAPE;
  if (((uintptr_t)out & 3) != 0) return NVFP4_ERR_ALIGN;
  hipLaunchKernelGGL(nvfp4::k_probe_philox, dim3(nvfp4::kProbeBlocks * 4), dim3(nvfp4::kProbeThreads), 0,
                     (hipStream_t)hip_stream, calls, (uint64_t)0x5EED, out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

extern "C" int nvfp4_probe_mfma(int64_t iters, float *out, void *hip_stream) {
  if (!out) return NVFP4_ERR_NULL;
  if (iters < 0) return NVFP4_ERR_SHAPE;
  if (((uintptr_t)out & 3) != 0) return NVFP4_ERR_ALIGN;
  hipLaunchKernelGGL(nvfp4::k_probe_mfma, dim3(nvfp4::kProbeBlocks), dim3(nvfp4::kProbeThreads), 0,
                     (hipStream_t)hip_stream, iters, out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}
