// Gate and top-k of one token per wave: the device functions shared by the
// router kernels (route.hip) and the fused routing + dispatch kernels.
//
// Sources: niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", sections
// "路由器怎样选专家：top-k 与两种门控" (softmax / sigmoid gate, top-k,
// renormalisation, routed_scaling_factor) and "DeepSeek-V3 的无辅助损失偏置"
// (selection-only expert bias, group-limited top-k).
#pragma once

#include <math.h>

#include "common.h"

namespace moe {
namespace {

// Wave-wide reductions without LDS traffic: four DPP steps leave every lane
// of a 16-lane row holding the row's result (swap neighbours, swap pairs,
// rotate the row by 4, then by 8, so each lane has met all four quads of its
// row), then lanes 0, 16, 32 and 48 are read into scalar registers and
// combined in a fixed order.  Every lane gets the same result.  The calling
// wave must have all 64 lanes active.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppRor4>(v);
  v += dpp_f<kDppRor8>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppRor4>(v));
  v = fmaxf(v, dpp_f<kDppRor8>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
// (v, i) pairs: the larger value wins, equal values -> the lower index.
__device__ __forceinline__ void argmax_pick(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& v, int& i) {
  argmax_pick(v, i, dpp_f<CTRL>(v), dpp_i<CTRL>(i));
}
// Larger value wins; equal values -> lower expert index.  v and i end up
// wave-uniform.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_dpp<kDppXor1>(v, i);
  argmax_dpp<kDppXor2>(v, i);
  argmax_dpp<kDppRor4>(v, i);
  argmax_dpp<kDppRor8>(v, i);
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < kWave; r += 16) argmax_pick(bv, bi, lane_f(v, r), __builtin_amdgcn_readlane(i, r));
  v = bv;
  i = bi;
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppRor4>(v));
  v = min(v, dpp_i<kDppRor8>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// A lane's N (value, index) pairs ordered best first: larger value, equal values
// -> lower index (insertion sort on a compile-time length).
template <int N>
__device__ __forceinline__ void sort_best_first(float (&v)[N], int (&i)[N]) {
#pragma unroll
  for (int a = 1; a < N; ++a)
#pragma unroll
    for (int b = a; b > 0; --b) {
      const bool sw = v[b] > v[b - 1] || (v[b] == v[b - 1] && i[b] < i[b - 1]);
      const float tv = sw ? v[b] : v[b - 1];
      const int ti = sw ? i[b] : i[b - 1];
      v[b] = sw ? v[b - 1] : v[b];
      i[b] = sw ? i[b - 1] : i[b];
      v[b - 1] = tv;
      i[b - 1] = ti;
    }
}

// The wave's best (value, index) among every lane's head pair (hv, hi): the
// largest value, then the lowest index; uniform.  The value is a plain wave
// maximum; the lane holding it is read from a ballot, and only exact ties of
// the maximum across lanes take a wave minimum over their indices.
__device__ __forceinline__ void wave_best_head(float hv, int hi, float& bv, int& bi) {
  const float m = wave_max(hv);
  const uint64_t match = __ballot(hv == m);
  if (__popcll(match) == 1)
    bi = __builtin_amdgcn_readlane(hi, (int)__builtin_ctzll(match));
  else
    bi = wave_min_i(hv == m ? hi : 0x7fffffff);
  bv = m;
}

// Options of the DeepSeek-V3 selection: selection-only bias and group limit.
struct SelOpts {
  const float* sbias;  // [E] or NULL
  int n_group;         // 0: no groups
  int topk_group;
  float* wbuf;         // this wave's LDS scratch of E floats (used when n_group > 0)
};

// Gate score of every expert of one token (one wave), the same arithmetic as
// the selection below: softmax over the E logits, or a sigmoid per logit.
template <int VPL>
__device__ void write_scores(const float (&z)[VPL], int E, int gate, float* out) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY, den = 0.f;
  if (gate == MOE_GATE_SOFTMAX) {
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (lane + kWave * v < E) m = fmaxf(m, z[v]);
    m = wave_max(m);
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (lane + kWave * v < E) den += expf(z[v] - m);
    den = wave_sum(den);
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane + kWave * v;
    if (e < E) out[e] = gate == MOE_GATE_SOFTMAX ? expf(z[v] - m) / den : 1.f / (1.f + expf(-z[v]));
  }
}

// Gate + top-k of one token, run by one whole wave.  z[v] holds the logit of
// expert lane + 64 v (-inf past E).
//  * Plain selection: both gates are increasing functions of z, so the k best
//    scores are the k largest logits; selection is done on z, which keeps full
//    fp32 resolution.
//  * With a selection bias or groups ([MoE-10] "DeepSeek-V3 的无辅助损失偏置"):
//    experts are ranked by gate score + bias, groups by the sum of their two
//    best ranking scores, only the topk_group best groups stay eligible, and
//    the weights are the unbiased scores of the picks.
// Ties go to the lower expert (or group) index.  Lanes j < k write pick j.
template <int VPL>
__device__ void topk_token(float (&z)[VPL], int E, int k, int gate, int renorm, float scale, const SelOpts& o,
                           float* out_scores, int32_t* out_idx, float* out_w) {
  const int lane = threadIdx.x & (kWave - 1);
  if (out_scores != nullptr) write_scores<VPL>(z, E, gate, out_scores);
  const bool plain = o.sbias == nullptr && o.n_group == 0;
  bool taken[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) taken[v] = false;
  float selz = -INFINITY, selsc = 0.f;
  int seli = 0;

  if (plain) {
    if constexpr (VPL <= 8) {
      // every lane orders its own logits best first once; each round takes the
      // wave's best head and the lane that held it moves on to its next one
      float hv[VPL];
      int hi[VPL];
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = lane + kWave * v;
        hv[v] = e < E ? z[v] : -INFINITY;
        hi[v] = e < E ? e : 0x7fffffff;
      }
      sort_best_first<VPL>(hv, hi);
      for (int j = 0; j < k; ++j) {
        float bv;
        int bi;
        wave_best_head(hv[0], hi[0], bv, bi);
        const bool pop = hi[0] == bi;
#pragma unroll
        for (int v = 0; v + 1 < VPL; ++v) {
          hv[v] = pop ? hv[v + 1] : hv[v];
          hi[v] = pop ? hi[v + 1] : hi[v];
        }
        if (pop) {
          hv[VPL - 1] = -INFINITY;
          hi[VPL - 1] = 0x7fffffff;
        }
        if (lane == j) { selz = bv; seli = bi; }
      }
    } else {
      for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          const int e = lane + kWave * v;
          if (e < E && !taken[v] && (z[v] > bv || bi == 0x7fffffff)) { bv = z[v]; bi = e; }
        }
        wave_argmax(bv, bi);
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (lane + kWave * v == bi) taken[v] = true;
        if (lane == j) { selz = bv; seli = bi; }
      }
    }
    const bool mine = lane < k;
    float w;
    if (gate == MOE_GATE_SOFTMAX) {
      if (renorm) {
        // p_j / sum_sel p = exp(z_j - z_best) / sum_sel exp(z - z_best)
        const float zbest = lane_f(selz, 0);
        const float ex = mine ? expf(selz - zbest) : 0.f;
        w = ex / wave_sum(ex);
      } else {
        // full softmax over all E experts
        float m = -INFINITY;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (lane + kWave * v < E) m = fmaxf(m, z[v]);
        m = wave_max(m);
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (lane + kWave * v < E) s += expf(z[v] - m);
        s = wave_sum(s);
        w = mine ? expf(selz - m) / s : 0.f;
      }
    } else {
      const float sg = mine ? 1.f / (1.f + expf(-selz)) : 0.f;
      w = renorm ? sg / wave_sum(sg) : sg;
    }
    if (mine) {
      out_idx[lane] = seli;
      out_w[lane] = w * scale;
    }
    return;
  }

  // ---- DeepSeek-V3 selection ----
  float m = -INFINITY, den = 0.f;
  if (gate == MOE_GATE_SOFTMAX) {
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (lane + kWave * v < E) m = fmaxf(m, z[v]);
    m = wave_max(m);
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (lane + kWave * v < E) den += expf(z[v] - m);
    den = wave_sum(den);
  }
  float sc[VPL], sel[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane + kWave * v;
    if (e < E) {
      sc[v] = gate == MOE_GATE_SOFTMAX ? expf(z[v] - m) / den : 1.f / (1.f + expf(-z[v]));
      sel[v] = o.sbias != nullptr ? sc[v] + o.sbias[e] : sc[v];
    } else {
      sc[v] = 0.f;
      sel[v] = -INFINITY;
    }
  }
  if (o.n_group > 0) {
    const int G = E / o.n_group;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + kWave * v;
      if (e < E) o.wbuf[e] = sel[v];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's scratch writes are done
    __builtin_amdgcn_wave_barrier();
    float gs = -INFINITY;
    if (lane < o.n_group) {  // group score: sum of its two best ranking scores
      float b1 = -INFINITY, b2 = -INFINITY;
      for (int i = 0; i < G; ++i) {
        const float v = o.wbuf[lane * G + i];
        if (v > b1) { b2 = b1; b1 = v; }
        else if (v > b2) b2 = v;
      }
      gs = G >= 2 ? b1 + b2 : b1;
    }
    uint64_t kept = 0;
    for (int q = 0; q < o.topk_group; ++q) {
      const bool cand = lane < o.n_group && !((kept >> lane) & 1);
      float bv = cand ? gs : -INFINITY;
      int bi = cand ? lane : 0x7fffffff;
      wave_argmax(bv, bi);
      if (bi < 64) kept |= 1ull << bi;  // always a group id when topk_group <= n_group
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + kWave * v;
      if (e < E && !((kept >> (e / G)) & 1)) sel[v] = -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();  // scratch reads done before a later token's writes
  }
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY, cs = 0.f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + kWave * v;
      if (e < E && !taken[v] && (sel[v] > bv || bi == 0x7fffffff)) { bv = sel[v]; bi = e; cs = sc[v]; }
    }
    wave_argmax(bv, bi);
    const float wsc = lane_f(cs, bi & (kWave - 1));  // the owner's local best is the winner (bi is uniform)
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (lane + kWave * v == bi) taken[v] = true;
    if (lane == j) { selsc = wsc; seli = bi; }
  }
  const bool mine = lane < k;
  const float w0 = mine ? selsc : 0.f;
  const float w = renorm ? w0 / wave_sum(w0) : w0;
  if (mine) {
    out_idx[lane] = seli;
    out_w[lane] = w * scale;
  }
}

}  // namespace
}  // namespace moe
