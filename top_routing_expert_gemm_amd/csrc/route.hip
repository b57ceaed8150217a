// Router GEMM fused with the gate and the top-k selection (gfx950).
//
// Sources: niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", sections
// "把一个大 FFN 换成一组小 FFN" (router = one linear layer x @ W_router.T) and
// "路由器怎样选专家：top-k 与两种门控" (softmax / sigmoid gate, top-k,
// renormalisation, routed_scaling_factor); amazingdata.cn "moe-routing-hardest"
// (the routing steps).
//
// bf16 path: one workgroup = 32 tokens x all E experts.  The 32 x 64 token tile is
// staged in LDS (double buffered, XOR-swizzled 16-byte chunks) and shared by the
// four waves; each wave streams its own 32-expert blocks of W_router straight
// into MFMA operand registers and accumulates z = x . W^T with
// v_mfma_f32_32x32x16_bf16 in fp32.  The logits tile goes to LDS only; each wave
// then runs the gate and top-k for 8 tokens with wave-wide reductions and writes
// just topk_idx / topk_w.
#include <math.h>

#include "common.h"

namespace moe {
namespace {

constexpr int kRBM = 32;   // tokens per workgroup
constexpr int kRBK = 64;   // K step
constexpr int kRThreads = 256;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
// Larger value wins; equal values -> lower expert index.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float v2 = __shfl_xor(v, off, kWave);
    int i2 = __shfl_xor(i, off, kWave);
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
  }
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
    const bool mine = lane < k;
    float w;
    if (gate == MOE_GATE_SOFTMAX) {
      if (renorm) {
        // p_j / sum_sel p = exp(z_j - z_best) / sum_sel exp(z - z_best)
        const float zbest = __shfl(selz, 0, kWave);
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
    const float wsc = __shfl(cs, bi & (kWave - 1), kWave);  // the owner's local best is the winner
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

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Router GEMM core shared by the fused and the split-K kernels: RBT blocks of
// 32 tokens (rows t0 ..) x all E experts, contraction over x columns
// [kb*64, ke*64).  The token tile is staged in LDS (As: 2 x RBT*32 x 64 bf16,
// double buffered, 16-byte chunks XOR-swizzled by row); each wave streams its
// 32-expert blocks of W_router straight into MFMA operand registers.
template <int NBW, int RBT>
__device__ __forceinline__ void router_tile(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T,
                                            int H, int E, int t0, int kb, int ke, uint16_t* As,
                                            f32x16 (&acc)[RBT][NBW], bool (&bval)[NBW]) {
  const int nblk = (E + 31) / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int ROWS = RBT * kRBM;

  // token tile staging: thread -> (row tid/8 + 32 i, 16-byte chunk tid%8)
  const int ar = tid >> 3, ac = tid & 7;
  const uint16_t* aptr[RBT];
  int a_lds[RBT];
#pragma unroll
  for (int i = 0; i < RBT; ++i) {
    const int r = ar + 32 * i;
    aptr[i] = x + (int64_t)min(t0 + r, T - 1) * H + ac * 8;
    a_lds[i] = r * kRBK + ((ac ^ (r & 7)) * 8);
  }
  // B operand rows of this wave's blocks: lane -> expert (lane & 31), k half (lane >> 5)
  const uint16_t* bptr[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int blk = wave + 4 * i;
    bval[i] = blk < nblk;
    const int e = min(blk * 32 + (lane & 31), E - 1);
    bptr[i] = w + (int64_t)e * H + (lane >> 5) * 32;
  }
#pragma unroll
  for (int r = 0; r < RBT; ++r)
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[r][i][v] = 0.f;

  uint4 apf[RBT];
  uint4 bcur[NBW][4];
#pragma unroll
  for (int i = 0; i < RBT; ++i) apf[i] = ldg16(aptr[i] + kb * kRBK);
#pragma unroll
  for (int i = 0; i < NBW; ++i)
    if (bval[i])
#pragma unroll
      for (int s = 0; s < 4; ++s) bcur[i][s] = ldg16(bptr[i] + kb * kRBK + s * 8);
#pragma unroll
  for (int i = 0; i < RBT; ++i) *reinterpret_cast<uint4*>(As + a_lds[i]) = apf[i];
  __syncthreads();

  const int arow = lane & 31;
  for (int kt = kb; kt < ke; ++kt) {
    uint4 bnext[NBW][4];
    const bool more = kt + 1 < ke;
    if (more) {
#pragma unroll
      for (int i = 0; i < RBT; ++i) apf[i] = ldg16(aptr[i] + (kt + 1) * kRBK);
#pragma unroll
      for (int i = 0; i < NBW; ++i)
        if (bval[i])
#pragma unroll
          for (int s = 0; s < 4; ++s) bnext[i][s] = ldg16(bptr[i] + (kt + 1) * kRBK + s * 8);
    }
    const uint16_t* Ab = As + ((kt - kb) & 1) * ROWS * kRBK;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // substep s, lane half h: k = h*32 + s*8 .. +8 (same permutation as the B loads)
      const int chunk = (lane >> 5) * 4 + s;
#pragma unroll
      for (int r = 0; r < RBT; ++r) {
        const int row = r * 32 + arow;
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(Ab + row * kRBK + ((chunk ^ (row & 7)) * 8)));
#pragma unroll
        for (int i = 0; i < NBW; ++i)
          if (bval[i])
            acc[r][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, bcur[i][s]),
                                                                acc[r][i], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < RBT; ++i)
        *reinterpret_cast<uint4*>(As + (((kt - kb) + 1) & 1) * ROWS * kRBK + a_lds[i]) = apf[i];
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s) bcur[i][s] = bnext[i][s];
    }
    __syncthreads();
  }
}

// Fused router: one workgroup = 32 tokens x all E experts over the whole of H;
// logits go to LDS only, then each wave runs the gate / top-k of 8 tokens.
template <int NBW>
__global__ __launch_bounds__(kRThreads) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const float* __restrict__ bias,
    int T, int H, int E, int k, int gate, int renorm, float scale, RouteSel rs, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  constexpr int VPL = 2 * NBW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);                 // [2][32][64] bf16
  float* lg = reinterpret_cast<float*>(smem + 2 * kRBM * kRBK * 2);  // [32][lde]
  const int nblk = (E + 31) / 32;
  const int lde = nblk * 32 + 4;
  float* wscr = lg + kRBM * lde;                                     // [4][nblk*32] group scratch
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRBM;

  f32x16 acc[1][NBW];
  bool bval[NBW];
  router_tile<NBW, 1>(x, w, T, H, E, t0, 0, H / kRBK, As, acc, bval);

  // logits tile -> LDS: lane holds expert column (lane & 31) of each block and
  // token rows 8g + 4*(lane >> 5) + r of the 32x32 MFMA result.
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    if (!bval[i]) continue;
    const int e = (wave + 4 * i) * 32 + (lane & 31);
    const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 8 * g + 4 * (lane >> 5) + r;
        lg[row * lde + e] = acc[0][i][4 * g + r] + b;
      }
  }
  __syncthreads();

  const SelOpts o{rs.sbias, rs.n_group, rs.topk_group, wscr + wave * nblk * 32};
  for (int row = wave; row < kRBM; row += 4) {
    const int t = t0 + row;
    if (t >= T) break;
    float z[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + kWave * v;
      z[v] = e < E ? lg[row * lde + e] : -INFINITY;
    }
    topk_token<VPL>(z, E, k, gate, renorm, scale, o, rs.scores ? rs.scores + (int64_t)t * E : nullptr, topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k);
  }
}

// Split-K router, part 1: workgroup (m, s) computes the partial logits of RBT*32
// tokens over the s-th slice of H and stores them to part[s][t][0..Epad).  The
// 128-token tiles of the largest batches are held to two waves per SIMD (within
// 256 VGPRs), so two workgroups share a CU and hide each other's load latency.
template <int NBW, int RBT>
__global__ __launch_bounds__(kRThreads) __attribute__((amdgpu_waves_per_eu(RBT == 4 ? 2 : 1))) void route_partial_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int H, int E, int ksteps_per_split,
    float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2 * RBT * kRBM * kRBK];
  const int nblk = (E + 31) / 32, Epad = nblk * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * RBT * kRBM;
  const int ks = blockIdx.y;
  const int kb = ks * ksteps_per_split;
  const int ke = min(kb + ksteps_per_split, H / kRBK);
  f32x16 acc[RBT][NBW];
  bool bval[NBW];
  router_tile<NBW, RBT>(x, w, T, H, E, t0, kb, ke, As, acc, bval);
  float* out = part + (int64_t)ks * T * Epad;
#pragma unroll
  for (int r = 0; r < RBT; ++r)
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      if (!bval[i]) continue;
      const int e = (wave + 4 * i) * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = t0 + r * 32 + 8 * g + 4 * (lane >> 5) + q;
          if (t < T) out[(int64_t)t * Epad + e] = acc[r][i][4 * g + q];
        }
    }
}

// Split-K router, part 2: one wave per token sums the partial logits in slice
// order (fixed, so the result is reproducible), adds the bias and runs the gate
// and top-k.
template <int VPL>
__global__ __launch_bounds__(kRThreads) void route_topk_kernel(const float* __restrict__ part, int nsplit, int T,
                                                               int E, const float* __restrict__ bias, int k,
                                                               int gate, int renorm, float scale,
                                                               RouteSel rs, int32_t* __restrict__ topk_idx,
                                                               float* __restrict__ topk_w) {
  constexpr int TPB = kRThreads / kWave;  // tokens per workgroup, one wave each for the top-k
  // dynamic LDS sized by E (topk_lds_bytes): the summed logits of the TPB tokens, then each wave's group
  // scratch, E floats each, so a small E leaves room for more workgroups per CU
  extern __shared__ __attribute__((aligned(16))) float tk_lds[];
  float* zs = tk_lds;                 // [TPB][E]
  float* wscr = tk_lds + TPB * E;     // [TPB][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TPB;
  const int Epad = (E + 31) / 32 * 32;
  const int64_t stride = (int64_t)T * Epad;
  // The whole workgroup sums the slice partials of its TPB tokens: thread -> expert,
  // all tokens at once, eight slices per round, added strictly in slice order.
  for (int e = threadIdx.x; e < E; e += kRThreads) {
    float s[TPB];
#pragma unroll
    for (int j = 0; j < TPB; ++j) s[j] = 0.f;
    const float* pp = part + (int64_t)t0 * Epad + e;
    int ks = 0;
    for (; ks + 8 <= nsplit; ks += 8) {
      float q[8][TPB];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < TPB; ++j) q[u][j] = t0 + j < T ? pp[(ks + u) * stride + (int64_t)j * Epad] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < TPB; ++j) s[j] += q[u][j];
    }
    if (ks < nsplit) {  // the last < 8 slices: loads issued together, then added in slice order
      float q[8][TPB];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < TPB; ++j)
          q[u][j] = (ks + u < nsplit && t0 + j < T) ? pp[(ks + u) * stride + (int64_t)j * Epad] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (ks + u < nsplit)
#pragma unroll
          for (int j = 0; j < TPB; ++j) s[j] += q[u][j];
    }
#pragma unroll
    for (int j = 0; j < TPB; ++j) zs[j * E + e] = s[j];
  }
  __syncthreads();
  const int t = t0 + wave;
  if (t >= T) return;
  float z[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane + kWave * v;
    z[v] = e < E ? (bias != nullptr ? zs[wave * E + e] + bias[e] : zs[wave * E + e]) : -INFINITY;
  }
  const SelOpts o{rs.sbias, rs.n_group, rs.topk_group, wscr + wave * E};
  topk_token<VPL>(z, E, k, gate, renorm, scale, o, rs.scores ? rs.scores + (int64_t)t * E : nullptr,
                  topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k);
}

// fp32 path: one wave per token computes its E logits with lane-strided dot
// products and a fixed-order wave reduction, then runs the same gate / top-k.
template <int VPL>
__global__ __launch_bounds__(kRThreads) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias, int T,
    int H, int E, int k, int gate, int renorm, float scale, RouteSel rs, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  __shared__ float wscr[kRThreads / kWave][kMaxE];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kRThreads / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)t * H);
  float z[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    z[v] = -INFINITY;
    for (int el = 0; el < kWave; ++el) {
      const int e = v * kWave + el;
      if (e >= E) break;
      const float4* wr = reinterpret_cast<const float4*>(w + (int64_t)e * H);
      float s = 0.f;
      for (int h4 = lane; h4 < H / 4; h4 += kWave) {
        const float4 a = xr[h4], b = wr[h4];
        s = fmaf(a.x, b.x, s);
        s = fmaf(a.y, b.y, s);
        s = fmaf(a.z, b.z, s);
        s = fmaf(a.w, b.w, s);
      }
      s = wave_sum(s);
      if (bias != nullptr) s += bias[e];
      if (lane == el) z[v] = s;
    }
  }
  const SelOpts o{rs.sbias, rs.n_group, rs.topk_group, wscr[threadIdx.x >> 6]};
  topk_token<VPL>(z, E, k, gate, renorm, scale, o, rs.scores ? rs.scores + (int64_t)t * E : nullptr, topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k);
}

template <int NBW>
hipError_t launch_route_bf16(const moe_config& c, const void* x, const void* w, const float* bias,
                             const RouteSel& rs, int32_t* idx, float* tw, hipStream_t s) {
  const int nblk = (int)((c.E + 31) / 32);
  const size_t lds = 2 * kRBM * kRBK * 2 + (size_t)kRBM * (nblk * 32 + 4) * 4 + (size_t)4 * nblk * 32 * 4;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_bf16_kernel<NBW>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int grid = (int)((c.T + kRBM - 1) / kRBM);
  hipLaunchKernelGGL(route_bf16_kernel<NBW>, dim3(grid), dim3(kRThreads), lds, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), bias, (int)c.T,
                     (int)c.H, (int)c.E, (int)c.k, c.gate, c.renormalize, c.routed_scaling_factor, rs, idx, tw);
  return hipGetLastError();
}

template <int VPL>
hipError_t launch_route_f32(const moe_config& c, const void* x, const void* w, const float* bias,
                            const RouteSel& rs, int32_t* idx, float* tw, hipStream_t s) {
  const int per = kRThreads / kWave;
  const int grid = (int)((c.T + per - 1) / per);
  hipLaunchKernelGGL(route_f32_kernel<VPL>, dim3(grid), dim3(kRThreads), 0, s,
                     static_cast<const float*>(x), static_cast<const float*>(w), bias, (int)c.T,
                     (int)c.H, (int)c.E, (int)c.k, c.gate, c.renormalize, c.routed_scaling_factor, rs, idx, tw);
  return hipGetLastError();
}

// Token blocks per workgroup: 128 tokens for the largest batches with E <= 256
// and 64 for large ones (fewer passes over the router weights per token), 32
// otherwise and for E > 512 (register budget).
// Split factor of the K dimension: enough workgroups to cover the chip twice
// (two 128-token workgroups fit per CU), each slice at least four K steps long.
inline int route_rbt(int64_t T, int64_t E) {
  if (T >= 8192 && E <= 256) return 4;
  return T >= 4096 && E <= 512 ? 2 : 1;
}
inline int route_nsplit(int64_t T, int64_t H, int64_t E) {
  const int rbt = route_rbt(T, E);
  const int64_t rows = rbt * kRBM;
  const int64_t mt = (T + rows - 1) / rows;
  const int64_t nk = H / kRBK;
  const int64_t target = 512;
  int64_t ns = (target + mt - 1) / mt;
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, nk / 4));
  return (int)std::max<int64_t>(1, ns);
}

template <int NBW, int RBT>
hipError_t launch_route_split_t(const moe_config& c, const void* x, const void* w, const float* bias,
                                const RouteSel& rs, int32_t* idx, float* tw, float* part, hipStream_t s) {
  const int nsplit = route_nsplit(c.T, c.H, c.E);
  const int nk = (int)(c.H / kRBK);
  const int per = (nk + nsplit - 1) / nsplit;
  const int nsplit_eff = (nk + per - 1) / per;
  dim3 grid((unsigned)((c.T + RBT * kRBM - 1) / (RBT * kRBM)), (unsigned)nsplit_eff);
  hipLaunchKernelGGL((route_partial_bf16_kernel<NBW, RBT>), grid, dim3(kRThreads), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), (int)c.T, (int)c.H,
                     (int)c.E, per, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tpb = kRThreads / kWave;
  const size_t lds = (size_t)2 * tpb * c.E * sizeof(float);
  hipLaunchKernelGGL(route_topk_kernel<2 * NBW>, dim3((unsigned)((c.T + tpb - 1) / tpb)), dim3(kRThreads), lds, s,
                     part, nsplit_eff, (int)c.T, (int)c.E, bias, (int)c.k, c.gate, c.renormalize,
                     c.routed_scaling_factor, rs, idx, tw);
  return hipGetLastError();
}

template <int NBW>
hipError_t launch_route_split_n(const moe_config& c, const void* x, const void* w, const float* bias,
                                const RouteSel& rs, int32_t* idx, float* tw, float* part, hipStream_t s) {
  if constexpr (NBW <= 2)
    if (route_rbt(c.T, c.E) == 4) return launch_route_split_t<NBW, 4>(c, x, w, bias, rs, idx, tw, part, s);
  if constexpr (NBW <= 4)
    if (route_rbt(c.T, c.E) == 2) return launch_route_split_t<NBW, 2>(c, x, w, bias, rs, idx, tw, part, s);
  return launch_route_split_t<NBW, 1>(c, x, w, bias, rs, idx, tw, part, s);
}

}  // namespace

size_t route_scratch_bytes(const moe_config& c) {
  if (c.dtype != MOE_BF16) return 0;
  const int64_t Epad = (c.E + 31) / 32 * 32;
  return (size_t)route_nsplit(c.T, c.H, c.E) * c.T * Epad * 4;
}

hipError_t launch_route_split(const moe_config& c, const void* x, const void* w, const float* bias,
                              const RouteSel& rs, int32_t* topk_idx, float* topk_w, void* scratch,
                              hipStream_t s) {
  if (c.dtype != MOE_BF16) return launch_route(c, x, w, bias, rs, topk_idx, topk_w, s);
  float* part = static_cast<float*>(scratch);
  if (c.E <= 128) return launch_route_split_n<1>(c, x, w, bias, rs, topk_idx, topk_w, part, s);
  if (c.E <= 256) return launch_route_split_n<2>(c, x, w, bias, rs, topk_idx, topk_w, part, s);
  if (c.E <= 512) return launch_route_split_n<4>(c, x, w, bias, rs, topk_idx, topk_w, part, s);
  return launch_route_split_n<8>(c, x, w, bias, rs, topk_idx, topk_w, part, s);
}

hipError_t launch_route(const moe_config& c, const void* x, const void* w, const float* bias, const RouteSel& rs,
                        int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (c.dtype == MOE_BF16) {
    if (c.E <= 128) return launch_route_bf16<1>(c, x, w, bias, rs, topk_idx, topk_w, s);
    if (c.E <= 256) return launch_route_bf16<2>(c, x, w, bias, rs, topk_idx, topk_w, s);
    if (c.E <= 512) return launch_route_bf16<4>(c, x, w, bias, rs, topk_idx, topk_w, s);
    return launch_route_bf16<8>(c, x, w, bias, rs, topk_idx, topk_w, s);
  }
  if (c.E <= 64) return launch_route_f32<1>(c, x, w, bias, rs, topk_idx, topk_w, s);
  if (c.E <= 256) return launch_route_f32<4>(c, x, w, bias, rs, topk_idx, topk_w, s);
  return launch_route_f32<16>(c, x, w, bias, rs, topk_idx, topk_w, s);
}

}  // namespace moe
