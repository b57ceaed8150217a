// Load-balancing statistics of one routed batch and the selection-bias step.
//
// Sources: niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", section "辅助损失"
// (f_i = share of the batch's assignments that went to expert i, P_i = mean
// routing probability of expert i, balance term N * sum_i f_i P_i, 1 for a
// uniform router) and section "DeepSeek-V3 的无辅助损失偏置" (after each step an
// overloaded expert's selection bias drops by gamma, an underloaded one's rises
// by gamma).
//
// Both are tiny next to the layer: P_i is a column mean of the [T, E] score
// matrix (HBM-bound, T*E*4 bytes read once), the rest touches E values.
// Every sum runs in a fixed order (no atomics), so results are reproducible.
#include "common.h"

namespace moe {
namespace {

constexpr int kStatRows = 256;   // tokens per partial column sum
constexpr int kStatWaves = 8;    // waves per partial-sum workgroup
constexpr int kFinThreads = 1024;

// Pass 1: part[c][e] = sum over tokens r of chunk c of scores[r][e].  One
// workgroup covers 64 expert columns x kStatRows tokens; wave w sums rows
// w, w + 8, ... (each row is one coalesced 256-byte load of the wave), and the
// eight wave sums are added in wave order.
__global__ __launch_bounds__(kStatWaves * kWave) void score_partial_kernel(const float* __restrict__ scores, int T,
                                                                           int E, float* __restrict__ part) {
  __shared__ float red[kStatWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int e = blockIdx.y * kWave + lane;
  const int r0 = blockIdx.x * kStatRows;
  const int r1 = min(T, r0 + kStatRows);
  float s = 0.f;
  if (e < E) {
    const float* p = scores + (int64_t)r0 * E + e;
#pragma unroll 8
    for (int r = r0 + wave; r < r1; r += kStatWaves) s += p[(int64_t)(r - r0) * E];
  }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && e < E) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kStatWaves; ++w) t += red[w][lane];
    part[(int64_t)blockIdx.x * E + e] = t;
  }
}

// Pass 2 (one workgroup): P_e = (sum of the partials in chunk order) / T,
// f_e = counts[e] / (T k) (divided in double, rounded once to float), and the
// balance term E * sum_e f_e P_e: thread-local sums over e = tid, tid + 1024, ...,
// then a fixed tree over the threads.
__global__ __launch_bounds__(kFinThreads) void balance_final_kernel(const float* __restrict__ part, int nchunk,
                                                                    const int32_t* __restrict__ counts, int T, int E,
                                                                    int k, float* __restrict__ mean,
                                                                    float* __restrict__ frac,
                                                                    float* __restrict__ balance) {
  __shared__ float red[kFinThreads];
  const int tid = threadIdx.x;
  const double tk = (double)T * (double)k;
  float acc = 0.f;
  for (int e = tid; e < E; e += kFinThreads) {
    float s = 0.f;
    for (int c = 0; c < nchunk; ++c) s += part[(int64_t)c * E + e];
    const float P = s / (float)T;
    const float f = (float)((double)counts[e] / tk);
    if (mean != nullptr) mean[e] = P;
    if (frac != nullptr) frac[e] = f;
    acc += f * P;
  }
  red[tid] = acc;
  __syncthreads();
  for (int off = kFinThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  if (tid == 0 && balance != nullptr) balance[0] = (float)E * red[0];
}

// One workgroup: the mean load is sum(counts) / E, so "load below the mean" is
// the exact integer test counts[e] * E < sum(counts).  The bias moves by +-gamma
// in float32; an expert exactly at the mean keeps its bias.
__global__ __launch_bounds__(kFinThreads) void bias_update_kernel(const int32_t* __restrict__ counts, int E,
                                                                  float gamma, float* __restrict__ bias) {
  __shared__ long long red[kFinThreads];
  const int tid = threadIdx.x;
  long long own = 0;
  for (int e = tid; e < E; e += kFinThreads) own += counts[e];
  red[tid] = own;
  __syncthreads();
  for (int off = kFinThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const long long total = red[0];
  for (int e = tid; e < E; e += kFinThreads) {
    const long long scaled = (long long)counts[e] * E;
    if (scaled < total) bias[e] += gamma;
    else if (scaled > total) bias[e] -= gamma;
  }
}

inline int stat_chunks(int64_t T) { return (int)((T + kStatRows - 1) / kStatRows); }

}  // namespace

size_t stats_scratch_bytes(const moe_config& c) { return (size_t)stat_chunks(c.T) * c.E * sizeof(float); }

hipError_t launch_balance_stats(const moe_config& c, const int32_t* counts, const float* scores, float* mean,
                                float* frac, float* balance, void* part, hipStream_t s) {
  const int nchunk = stat_chunks(c.T);
  float* pp = static_cast<float*>(part);
  dim3 grid((unsigned)nchunk, (unsigned)((c.E + kWave - 1) / kWave));
  hipLaunchKernelGGL(score_partial_kernel, grid, dim3(kStatWaves * kWave), 0, s, scores, (int)c.T, (int)c.E, pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(balance_final_kernel, dim3(1), dim3(kFinThreads), 0, s, pp, nchunk, counts, (int)c.T,
                     (int)c.E, (int)c.k, mean, frac, balance);
  return hipGetLastError();
}

hipError_t launch_bias_update(const moe_config& c, const int32_t* counts, float gamma, float* score_bias,
                              hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(kFinThreads), 0, s, counts, (int)c.E, gamma, score_bias);
  return hipGetLastError();
}

}  // namespace moe
