// Deterministic gate-weighted combine back to token order (gfx950).
//
// Sources: hi-bin.com "MoE为什么只激活一部分专家", section "Router 怎样给 Token
// 选专家" (y_t is the weighted sum of the selected experts' outputs);
// niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", section
// "细粒度专家与共享专家" (the shared expert's output is added directly) and
// section "负载不均：路由坍缩与丢 token" (a dropped token skips the expert).
//
// Work item = (token, chunk of 256 16-byte column vectors), grid-stride, so a
// small batch still spreads over many workgroups.  The kept (row, weight) pairs
// of the token are read and compacted in slot order, then each thread
// accumulates one 16-byte column vector of those y_perm rows in float32 in slot
// order j = 0..k-1, adds the shared row, and stores.  A gather, not a scatter: no atomics, so the result is bitwise
// reproducible.  HBM bound: reads (kept slots + shared) rows, writes one row.  The row loads of a
// thread are issued kCombineBatch at a time before any is accumulated, so that the memory system has
// that many requests of each thread in flight rather than one.
#include "common.h"

namespace moe {
namespace {

constexpr int kCombineBatch = 8;

// Rows of y_perm and of the shared expert's output are read exactly once, each
// wave load a whole 1 KB piece of a row: non-temporal loads (a large buffer
// read this way streams at about 7.1 TB/s on this device, 6.2-6.3 TB/s
// without the hint).
#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1
#endif
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_once(const uint4* p) {
  if (MOE_COMBINE_NT) {
    const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  return *p;
}

__device__ __forceinline__ void acc_bf16x8(float (&acc)[8], const uint4& v, float w) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, __uint_as_float(u[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
  }
}

// The token's kept (row, weight) pairs, in slot order, into LDS: slots are read
// 256 at a time and compacted with wave ballots, so a token with k slots of
// which few are kept (expert choice: k = E) costs only its kept rows later.
// Returns the number of kept pairs; weights are multiplied by `scale`.
__device__ __forceinline__ int load_pairs(const int32_t* __restrict__ ros, const float* __restrict__ tw, int64_t t,
                                          int k, float scale, int* s_row, float* s_w, int* s_cnt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int n = 0;
  for (int j0 = 0; j0 < k; j0 += 256) {
    const int j = j0 + threadIdx.x;
    int row = -1;
    float w = 0.f;
    if (j < k) {  // both loads issued together; the weight is kept only for a kept slot
      row = ros[t * k + j];
      const float wj = tw[t * k + j];
      if (row >= 0) w = wj;
    }
    const uint64_t b = __ballot(row >= 0);
    if (lane == 0) s_cnt[wave] = __popcll(b);
    __syncthreads();
    int off = n, tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < wave) off += s_cnt[q];
      tot += s_cnt[q];
    }
    if (row >= 0) {
      const int at = off + __popcll(b & ((1ull << lane) - 1ull));
      s_row[at] = row;
      s_w[at] = w * scale;
    }
    n += tot;
    __syncthreads();
  }
  return n;
}

__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint16_t* __restrict__ yp,
                                                           const int32_t* __restrict__ ros,
                                                           const float* __restrict__ tw,
                                                           const uint16_t* __restrict__ ysh,
                                                           uint16_t* __restrict__ y, int64_t T, int64_t H, int k,
                                                           float scale) {
  __shared__ int s_row[kMaxE];
  __shared__ float s_w[kMaxE];
  __shared__ int s_cnt[4];
  const int64_t hv = H / 8;
  const int64_t nch = (hv + blockDim.x - 1) / blockDim.x;  // column chunks of a row
  for (int64_t wi = blockIdx.x; wi < T * nch; wi += gridDim.x) {
    const int64_t t = wi / nch;
    const int n = load_pairs(ros, tw, t, k, scale, s_row, s_w, s_cnt);
    const int64_t c = (wi % nch) * blockDim.x + threadIdx.x;
    if (c < hv) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
      const uint4 vsh = ysh != nullptr ? ld_once(reinterpret_cast<const uint4*>(ysh + t * H) + c) : uint4{0, 0, 0, 0};
      for (int j0 = 0; j0 < n; j0 += kCombineBatch) {
        uint4 v[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
          if (j0 + u < n) v[u] = ld_once(reinterpret_cast<const uint4*>(yp + (int64_t)s_row[j0 + u] * H) + c);
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
          if (j0 + u < n) acc_bf16x8(acc, v[u], s_w[j0 + u]);
      }
      if (ysh != nullptr) acc_bf16x8(acc, vsh, 1.f);
      uint4 o;
      o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
      o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
      o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
      o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
      reinterpret_cast<uint4*>(y + t * H)[c] = o;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ yp,
                                                          const int32_t* __restrict__ ros,
                                                          const float* __restrict__ tw,
                                                          const float* __restrict__ ysh, float* __restrict__ y,
                                                          int64_t T, int64_t H, int k, float scale) {
  __shared__ int s_row[kMaxE];
  __shared__ float s_w[kMaxE];
  __shared__ int s_cnt[4];
  const int64_t hv = H / 4;
  const int64_t nch = (hv + blockDim.x - 1) / blockDim.x;  // column chunks of a row
  for (int64_t wi = blockIdx.x; wi < T * nch; wi += gridDim.x) {
    const int64_t t = wi / nch;
    const int n = load_pairs(ros, tw, t, k, scale, s_row, s_w, s_cnt);
    const int64_t c = (wi % nch) * blockDim.x + threadIdx.x;
    if (c < hv) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 vsh = ysh != nullptr ? reinterpret_cast<const float4*>(ysh + t * H)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j0 = 0; j0 < n; j0 += kCombineBatch) {
        float4 v[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
          if (j0 + u < n) v[u] = reinterpret_cast<const float4*>(yp + (int64_t)s_row[j0 + u] * H)[c];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
          if (j0 + u < n) {
            const float w = s_w[j0 + u];
            acc.x = fmaf(w, v[u].x, acc.x);
            acc.y = fmaf(w, v[u].y, acc.y);
            acc.z = fmaf(w, v[u].z, acc.z);
            acc.w = fmaf(w, v[u].w, acc.w);
          }
      }
      if (ysh != nullptr) {
        const float4 v = vsh;
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
      reinterpret_cast<float4*>(y + t * H)[c] = acc;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_combine(const void* y_perm, const int32_t* row_of_slot, const float* topk_w,
                          const void* y_shared, void* y, int64_t T, int64_t H, int64_t k, int dtype,
                          hipStream_t s, float scale) {
  const int64_t hv = dtype == MOE_BF16 ? H / 8 : H / 4;
  const unsigned grid = (unsigned)std::min<int64_t>(T * ((hv + 255) / 256), 16384);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(grid), dim3(256), 0, s, static_cast<const uint16_t*>(y_perm),
                       row_of_slot, topk_w, static_cast<const uint16_t*>(y_shared), static_cast<uint16_t*>(y), T,
                       H, (int)k, scale);
  else
    hipLaunchKernelGGL(combine_f32_kernel, dim3(grid), dim3(256), 0, s, static_cast<const float*>(y_perm),
                       row_of_slot, topk_w, static_cast<const float*>(y_shared), static_cast<float*>(y), T, H,
                       (int)k, scale);
  return hipGetLastError();
}

}  // namespace moe
