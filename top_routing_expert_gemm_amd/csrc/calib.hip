// Calibration kernels (not part of the layer): the bf16 MFMA rate the device
// sustains with no memory traffic at all, and the rate at which it reads a
// large buffer from HBM with no arithmetic to speak of, to set the layer's
// kernels against what each side of the chip reaches on its own.
#include "common.h"

namespace moe {
namespace {

constexpr int kCalWG = 2048;       // workgroups (8 per CU)
constexpr int kCalThreads = 256;   // 4 waves
constexpr int kCalChains = 4;      // independent accumulator chains per wave

// Operand bits of the varied mode: set j (< 8), element i of lane l, a or b
// (ab = 0 / 1): a sign, an exponent of 2^-4 and a mantissa from an integer
// hash, so consecutive MFMAs see unrelated inputs, as a GEMM's operands are.
__device__ __forceinline__ uint16_t cal_bits(uint32_t lane, uint32_t j, uint32_t i, uint32_t ab) {
  uint32_t h = lane * 0x9E3779B1u ^ (j * 8u + i) * 0x85EBCA77u ^ ab * 0xC2B2AE3Du;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  return (uint16_t)(0x3D80u | (h & 0x807Fu));
}

// VARIED = false: every MFMA multiplies the same two register operands;
// VARIED = true: eight operand pairs in turn, so every MFMA's inputs differ
// from the previous one's (the matrix units toggle as on real data, which draws
// more power and can lower the clock the device holds).
template <bool VARIED>
__global__ __launch_bounds__(kCalThreads) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  constexpr int NS = VARIED ? 8 : 1;
  bf16x8 a[NS], b[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (VARIED) {
        a[j][i] = __builtin_bit_cast(__bf16, cal_bits(lane, j, i, 0));
        b[j][i] = __builtin_bit_cast(__bf16, cal_bits(lane, j, i, 1));
      } else {
        a[j][i] = (__bf16)(1e-3f * (float)((lane + i) & 7));
        b[j][i] = (__bf16)(1e-3f * (float)((lane * 3 + i) & 7));
      }
    }
  f32x16 acc[kCalChains];
#pragma unroll
  for (int c = 0; c < kCalChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
  if constexpr (VARIED) {
    // chain c: operand pair c on even iterations, pair 4 + c on odd ones
    int it = 0;
    for (; it + 1 < iters; it += 2) {
#pragma unroll
      for (int c = 0; c < kCalChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < kCalChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[4 + c], b[4 + c], acc[c], 0, 0, 0);
    }
    if (it < iters) {
#pragma unroll
      for (int c = 0; c < kCalChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kCalChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kCalChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  if (lane == 0) sink[blockIdx.x * (kCalThreads / kWave) + threadIdx.x / kWave] = s;
}

constexpr int kReadWG = 4096;                // workgroups of the read stream
constexpr int kReadThreads = 256;
constexpr int kReadLoads = 8;                // 16-byte loads per thread per block
static_assert(kReadThreads * kReadLoads * 16 == 32768, "one block is 32 KiB");

// Non-temporal loads: each wave load covers whole 128-byte lines, and with
// this hint a large buffer streams at about 7.1 TB/s on this device against
// 6.2-6.3 TB/s for plain loads (the lines are then not kept in the caches).
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void read_block(uint4 (&r)[kReadLoads], const uint4* __restrict__ p, int64_t b) {
  const uint4* q = p + b * (kReadThreads * kReadLoads) + threadIdx.x;
#pragma unroll
  for (int j = 0; j < kReadLoads; ++j) {
    const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(q + j * kReadThreads));
    r[j] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

__device__ __forceinline__ void xor_in(uint32_t& acc, const uint4 (&r)[kReadLoads]) {
#pragma unroll
  for (int j = 0; j < kReadLoads; ++j) acc ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
}

// Workgroup w reads the 32 KiB blocks w, w + kReadWG, w + 2 kReadWG, ... (each
// thread eight 16-byte vectors of a block, a block's loads one contiguous
// sweep), the next block's loads issued before the current one is folded in,
// and writes the XOR of every 32-bit word it read to sink[w].
__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const uint4* __restrict__ p, int64_t nblocks,
                                                               uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[kReadThreads / kWave];
  uint32_t acc = 0;
  uint4 a[kReadLoads], b[kReadLoads];
  int64_t blk = blockIdx.x;
  if (blk < nblocks) read_block(a, p, blk);
  for (; blk < nblocks; blk += 2 * kReadWG) {
    const bool has_b = blk + kReadWG < nblocks;
    if (has_b) read_block(b, p, blk + kReadWG);
    xor_in(acc, a);
    if (blk + 2 * kReadWG < nblocks) read_block(a, p, blk + 2 * kReadWG);
    if (has_b) xor_in(acc, b);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
#pragma unroll
    for (int w = 0; w < kReadThreads / kWave; ++w) v ^= part[w];
    sink[blockIdx.x] = v;
  }
}

}  // namespace

int64_t hbm_read_sink_len() { return kReadWG; }

hipError_t launch_hbm_read(const void* buf, int64_t nblocks, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(kReadWG), dim3(kReadThreads), 0, s, static_cast<const uint4*>(buf),
                     nblocks, sink);
  return hipGetLastError();
}

int64_t mfma_peak_flops(int64_t iters) {
  return (int64_t)kCalWG * (kCalThreads / kWave) * iters * kCalChains * (2LL * 32 * 32 * 16);
}

int64_t mfma_peak_sink_len() { return (int64_t)kCalWG * (kCalThreads / kWave); }

hipError_t launch_mfma_peak(int iters, bool varied, float* sink, hipStream_t s) {
  if (varied)
    hipLaunchKernelGGL(mfma_peak_kernel<true>, dim3(kCalWG), dim3(kCalThreads), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<false>, dim3(kCalWG), dim3(kCalThreads), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace moe
