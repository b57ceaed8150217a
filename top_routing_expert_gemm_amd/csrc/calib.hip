// Calibration kernel (not part of the layer): the bf16 MFMA rate the device
// sustains, to set the grouped GEMMs' measured rate against what the matrix
// cores reach with no memory traffic at all.
#include "common.h"

namespace moe {
namespace {

constexpr int kCalWG = 2048;       // workgroups (8 per CU)
constexpr int kCalThreads = 256;   // 4 waves
constexpr int kCalChains = 4;      // independent accumulator chains per wave

__global__ __launch_bounds__(kCalThreads) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)((lane + i) & 7));
    b[i] = (__bf16)(1e-3f * (float)((lane * 3 + i) & 7));
  }
  f32x16 acc[kCalChains];
#pragma unroll
  for (int c = 0; c < kCalChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kCalChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kCalChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  if (lane == 0) sink[blockIdx.x * (kCalThreads / kWave) + threadIdx.x / kWave] = s;
}

}  // namespace

int64_t mfma_peak_flops(int64_t iters) {
  return (int64_t)kCalWG * (kCalThreads / kWave) * iters * kCalChains * (2LL * 32 * 32 * 16);
}

int64_t mfma_peak_sink_len() { return (int64_t)kCalWG * (kCalThreads / kWave); }

hipError_t launch_mfma_peak(int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(kCalWG), dim3(kCalThreads), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace moe
