// Expert-choice selection (gfx950): every expert takes the C tokens with the
// highest gate score for it.
//
// Source: amazingdata.cn essay "moe-routing-hardest", the passage on the two
// routing schools: under expert choice each expert picks a fixed number of the
// tokens it wants most, which balances the load by construction and may leave
// some tokens with no expert.
//
// One workgroup per expert.  The C-th largest score of the expert's column is
// found exactly by a 4-pass radix select on order-preserving 32-bit keys
// (8 bits per pass, LDS histogram); then one pass in token order takes every
// token above that key and the first (C - #above) tokens equal to it, so equal
// scores go to the lower token id.  Outputs, all deterministic:
//   token_of_row[e*C + j]  the j-th chosen token of expert e (ascending token id)
//   row_of_pair[t*E + e]   its row e*C + j, or -1 when expert e did not take t.
#include "common.h"

namespace moe {
namespace {

constexpr int kEcThreads = 256;
constexpr int kEcWaves = kEcThreads / kWave;

// Float -> unsigned key with the same order (larger float, larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive count of `v` over the lower threads of the block, and the block total.
__device__ __forceinline__ int block_excl_count(bool v, int* s_cnt, int& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint64_t b = __ballot(v);
  const int below = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) s_cnt[wave] = __popcll(b);
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kEcWaves; ++w) {
    const int c = s_cnt[w];
    if (w < wave) off += c;
    total += c;
  }
  __syncthreads();  // s_cnt is reused by the next call
  return off + below;
}

__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(const float* __restrict__ scores, int T, int E, int C,
                                                               int32_t* __restrict__ token_of_row,
                                                               int32_t* __restrict__ row_of_pair) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_rem;
  __shared__ int s_cnt[kEcWaves];
  const int e = blockIdx.x, tid = threadIdx.x;
  const float* col = scores + e;

  // ---- radix select: key of the C-th largest score ----
  uint32_t prefix = 0, mask = 0;
  int rem = C;  // how many of the tokens matching `prefix` are still to take
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += kEcThreads) {
      const uint32_t key = order_key(col[(int64_t)t * E]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      // highest bucket b whose tokens, with those of every higher bucket, reach rem
      uint32_t above = 0;
      int b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= (uint32_t)rem) break;
        above += hist[b];
      }
      s_rem = rem - (int)above;
      s_prefix = prefix | ((uint32_t)b << shift);
      s_mask = mask | (0xffu << shift);
    }
    __syncthreads();
    prefix = s_prefix;
    mask = s_mask;
    rem = s_rem;
  }
  const uint32_t thr = prefix;  // exact key of the C-th largest score
  // rem = how many tokens with key == thr are taken (the lowest token ids)

  // ---- one pass in token order ----
  int taken = 0, eq_seen = 0;
  for (int t0 = 0; t0 < T; t0 += kEcThreads) {
    const int t = t0 + tid;
    uint32_t key = 0;
    if (t < T) key = order_key(col[(int64_t)t * E]);
    const bool gt = t < T && key > thr;
    const bool eq = t < T && key == thr;
    int n_eq;
    const int eq_rank = eq_seen + block_excl_count(eq, s_cnt, n_eq);
    const bool take = gt || (eq && eq_rank < rem);
    int n_take;
    const int pos = taken + block_excl_count(take, s_cnt, n_take);
    if (t < T) row_of_pair[(int64_t)t * E + e] = take ? e * C + pos : -1;
    if (take) token_of_row[(int64_t)e * C + pos] = t;
    taken += n_take;
    eq_seen += n_eq;
  }
}

}  // namespace

hipError_t launch_ec_select(const float* scores, int64_t T, int64_t E, int64_t C, int32_t* token_of_row,
                            int32_t* row_of_pair, hipStream_t s) {
  hipLaunchKernelGGL(ec_select_kernel, dim3((unsigned)E), dim3(kEcThreads), 0, s, scores, (int)T, (int)E, (int)C,
                     token_of_row, row_of_pair);
  return hipGetLastError();
}

}  // namespace moe
