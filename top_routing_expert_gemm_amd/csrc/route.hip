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
#include "topk.h"

namespace moe {
namespace {

constexpr int kRBM = 32;   // tokens per workgroup
constexpr int kRBK = 64;   // K step
constexpr int kRThreads = 256;

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row: the 16 lanes
// of one ds_read_b128 cycle (rows r .. r + 15, one logical chunk) land on
// distinct banks of the 64-bank LDS (rows r and r + 8 differ in the low bit).
__device__ __forceinline__ int rswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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
    a_lds[i] = r * kRBK + ((ac ^ rswz(r)) * 8);
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
            bf16x8, *reinterpret_cast<const uint4*>(Ab + row * kRBK + ((chunk ^ rswz(row)) * 8)));
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

// ------------------------------------------------------------------------
// Router partial logits of the layer path: part[s][t][0 .. Epad) = the logits of
// token t over the s-th slice of H (Epad = 32 ceil(E / 32); columns past E are
// not used).  The select step (dispatch.hip) adds the slices in slice order, so
// the sums are reproducible.

// Large batches, E <= 256: one workgroup = 256 tokens x all experts over one
// slice of H.  Four waves, one per SIMD; wave w computes tokens 64 w .. + 64 (two
// 32-row blocks) against every 32-expert block (NB of them), so the whole tile's
// 256 x 32 NB accumulators live in the workgroup's registers.  Both operand
// tiles go through LDS (double buffered, 128-byte rows, 16-byte chunks
// XOR-swizzled by row): every thread fetches the next K step's 16-byte pieces
// into registers while the current step is multiplied, then stores them; one
// barrier per step.  Per step the workgroup moves 32 KB of token rows and
// 4 NB KB of router weights for 256 x 32 NB x 64 multiply-adds: a 256-token
// tile reads the router weights once per 256 tokens, twice fewer times than
// 128-token tiles.
constexpr int kGT = 256;     // tokens per workgroup
constexpr int kGThreads = 256;

template <int NB>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void route_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int H, int E, int steps_per_split,
    float* __restrict__ part) {
  constexpr int EB = NB * 32;              // experts of the tile
  constexpr int NA = kGT * 8 / kGThreads;  // 16-byte A pieces per thread per step (8)
  constexpr int NBL = EB * 8 / kGThreads;  // B pieces per thread per step (NB)
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kGT * kRBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][EB * kRBK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kGT;
  const int ks = blockIdx.y;
  const int nk = H / kRBK;
  const int kb = ks * steps_per_split, ke = min(kb + steps_per_split, nk);
  const int Epad = (E + 31) / 32 * 32;

  // loader: thread -> row tid / 8 + 32 i, 16-byte chunk tid % 8 (stored at its swizzled slot)
  const int lr = tid >> 3, lc = tid & 7;
  const uint16_t* ap[NA];
  const uint16_t* bp[NBL];
  int aslot[NA], bslot[NBL];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = lr + 32 * i;
    ap[i] = x + (int64_t)min(t0 + r, T - 1) * H + lc * 8;
    aslot[i] = r * kRBK + ((lc ^ rswz(r)) * 8);
  }
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const int r = lr + 32 * i;
    bp[i] = w + (int64_t)min(r, E - 1) * H + lc * 8;
    bslot[i] = r * kRBK + ((lc ^ rswz(r)) * 8);
  }

  f32x16 acc[2][NB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][n][v] = 0.f;

  // two register sets: set P holds K step kt + 2 (issued during step kt), set
  // 1 - P step kt + 1 (issued during the previous step), stored to LDS at the
  // end of step kt; refills past the slice are clamped to its last step (loaded,
  // never used), so every step issues the same loads and the wait before each
  // store is an exact count
  uint4 ra[2][NA], rbv[2][NBL];
  auto load = [&](int set, int kt) {
    const int kc = min(kt, ke - 1) * kRBK;
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[set][i] = ldg16(ap[i] + kc);
#pragma unroll
    for (int i = 0; i < NBL; ++i) rbv[set][i] = ldg16(bp[i] + kc);
  };
  auto store = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<uint4*>(&sA[buf][aslot[i]]) = ra[set][i];
#pragma unroll
    for (int i = 0; i < NBL; ++i) *reinterpret_cast<uint4*>(&sB[buf][bslot[i]]) = rbv[set][i];
  };
  const int l32 = lane & 31, h = lane >> 5;
  auto compute = [&](int buf) {
    const uint16_t* A = sA[buf];
    const uint16_t* B = sB[buf];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      // substep s2, lane half h: k = 32 h + 8 s2 .. + 8 of the step, for A and B alike
      const int c = h * 4 + s2;
      bf16x8 av[2], bv[NB];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wave * 64 + j * 32 + l32;
        av[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(A + r * kRBK + ((c ^ rswz(r)) * 8)));
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int r = n * 32 + l32;
        bv[n] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(B + r * kRBK + ((c ^ rswz(r)) * 8)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[j][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[j], bv[n], acc[j][n], 0, 0, 0);
    }
  };
  load(0, kb);
  load(1, kb + 1);
  store(0, 0);
  __syncthreads();
  int kt = kb;
  for (; kt + 1 < ke; kt += 2) {  // the fences keep each refill issued before the step's MFMAs
    load(0, kt + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    store(1, 1);
    __syncthreads();
    load(1, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    store(0, 0);
    __syncthreads();
  }
  if (kt < ke) compute(0);

  // lane holds expert column l32 of each block and token rows 8 g + 4 h + q
  float* out = part + (int64_t)ks * T * Epad;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int e = n * 32 + l32;
      if (e >= Epad) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = t0 + wave * 64 + j * 32 + 8 * g + 4 * h + q;
          if (t < T) out[(int64_t)t * Epad + e] = acc[j][n][4 * g + q];
        }
    }
}

// Small batches (T <= 16): every workgroup owns 16 experts and one slice of H;
// its 16 waves split the slice's 64-wide K blocks between them (block i to wave
// i mod 16), stream the weight rows straight into registers (every block of a
// wave in flight at once) and multiply them with v_mfma_f32_16x16x32_bf16
// against the token rows (padded to 16 by repeating the last).  The waves'
// 16 x 16 partial logits are then added in LDS in wave order and written once
// per workgroup, so the select step reads only nsplit x T x E partials.
constexpr int kVWaves = 16;
constexpr int kVMaxBlk = 4;    // 64-wide K blocks per wave, at most

__global__ __launch_bounds__(kVWaves * 64) void route_gemv_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ w, int T, int H,
                                                                 int E, int nsplit, float* __restrict__ part) {
  __shared__ float red[kVWaves][16 * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = blockIdx.x, ks = blockIdx.y;
  const int nk = H / kRBK;
  const int kb = (int)((int64_t)ks * nk / nsplit), ke = (int)((int64_t)(ks + 1) * nk / nsplit);
  const int Epad = (E + 31) / 32 * 32;
  const int r16 = lane & 15, g4 = lane >> 4;
  // lane group g4 supplies k = 16 g4 .. + 16 of every 64-wide block, for A and B alike
  const uint16_t* pa = x + (int64_t)min(r16, T - 1) * H + g4 * 16;
  const uint16_t* pb = w + (int64_t)min(grp * 16 + r16, E - 1) * H + g4 * 16;
  uint4 a[kVMaxBlk][2], b[kVMaxBlk][2];
  int nb = 0;
#pragma unroll
  for (int i = 0; i < kVMaxBlk; ++i) {
    const int blk = kb + wave + kVWaves * i;
    if (blk < ke) {
      nb = i + 1;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        a[i][u] = ldg16(pa + blk * kRBK + 8 * u);
        b[i][u] = ldg16(pb + blk * kRBK + 8 * u);
      }
    }
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kVMaxBlk; ++i)
    if (i < nb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i][u]),
                                                      __builtin_bit_cast(bf16x8, b[i][u]), acc, 0, 0, 0);
  // lane holds expert column r16, token rows 4 g4 + q
#pragma unroll
  for (int q = 0; q < 4; ++q) red[wave][(4 * g4 + q) * 16 + r16] = acc[q];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int t = threadIdx.x >> 4, el = threadIdx.x & 15, e = grp * 16 + el;
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < kVWaves; ++v) s += red[v][threadIdx.x];
    if (t < T && e < E) part[((int64_t)ks * T + t) * Epad + e] = s;
  }
}

// Layers with E > 256 keep the 32-token-block tiles of the fused router: token
// blocks per workgroup 64 for large batches with E <= 512, 32 otherwise
// (register budget); K split so that the workgroups cover the chip twice, each
// slice at least four K steps long.
inline int route_rbt(int64_t T, int64_t E) { return T >= 4096 && E <= 512 ? 2 : 1; }
inline int route_nsplit_wide(int64_t T, int64_t H, int64_t E) {
  const int64_t rows = route_rbt(T, E) * kRBM;
  const int64_t mt = (T + rows - 1) / rows;
  const int64_t nk = H / kRBK;
  int64_t ns = (512 + mt - 1) / mt;
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, nk / 4));
  return (int)std::max<int64_t>(1, ns);
}

enum RouteKind { RK_GEMV = 0, RK_GEMM = 1, RK_WIDE = 2 };
struct RoutePlan {
  int kind;
  int nsplit;     // slices of H that hold partial logits
  int per;        // K steps per slice (RK_GEMM, RK_WIDE)
};

RoutePlan route_plan(const moe_config& c) {
  RoutePlan p{};
  const int nk = (int)(c.H / kRBK);
  if (c.T <= kGemvMaxT) {
    // about 64 workgroups in all, each slice at least one block per wave of half the waves
    p.kind = RK_GEMV;
    const int ngrp = (int)((c.E + 15) / 16);
    int ns = std::max(1, 64 / ngrp);
    ns = std::min(ns, std::max(1, nk / (kVWaves / 2)));
    ns = std::max(ns, (nk + kVWaves * kVMaxBlk - 1) / (kVWaves * kVMaxBlk));  // at most kVMaxBlk blocks per wave
    p.nsplit = ns;
    p.per = 0;
    return p;
  }
  if (c.E <= 256) {
    // one 256-token workgroup per CU in all, each slice at least four K steps long
    p.kind = RK_GEMM;
    const int64_t mt = (c.T + kGT - 1) / kGT;
    int64_t ns = (256 + mt - 1) / mt;
    ns = std::min<int64_t>(ns, std::max(1, nk / 4));
    p.per = (int)((nk + ns - 1) / ns);
    p.nsplit = (nk + p.per - 1) / p.per;
    return p;
  }
  p.kind = RK_WIDE;
  const int ns = route_nsplit_wide(c.T, c.H, c.E);
  p.per = (nk + ns - 1) / ns;
  p.nsplit = (nk + p.per - 1) / p.per;
  return p;
}

template <int NB>
hipError_t launch_route_gemm(const moe_config& c, const void* x, const void* w, int per, int nsplit, float* part,
                             hipStream_t s) {
  dim3 grid((unsigned)((c.T + kGT - 1) / kGT), (unsigned)nsplit);
  hipLaunchKernelGGL(route_gemm_kernel<NB>, grid, dim3(kGThreads), 0, s, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w), (int)c.T, (int)c.H, (int)c.E, per, part);
  return hipGetLastError();
}

template <int NBW, int RBT>
hipError_t launch_route_wide(const moe_config& c, const void* x, const void* w, int per, int nsplit, float* part,
                             hipStream_t s) {
  dim3 grid((unsigned)((c.T + RBT * kRBM - 1) / (RBT * kRBM)), (unsigned)nsplit);
  hipLaunchKernelGGL((route_partial_bf16_kernel<NBW, RBT>), grid, dim3(kRThreads), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), (int)c.T, (int)c.H,
                     (int)c.E, per, part);
  return hipGetLastError();
}

}  // namespace

int route_partial_slices(const moe_config& c) { return c.dtype == MOE_BF16 ? route_plan(c).nsplit : 0; }

size_t route_scratch_bytes(const moe_config& c) {
  if (c.dtype != MOE_BF16) return 0;
  const int64_t Epad = (c.E + 31) / 32 * 32;
  return (size_t)route_plan(c).nsplit * c.T * Epad * 4;
}

hipError_t launch_route_partials(const moe_config& c, const void* x, const void* w, float* part, hipStream_t s) {
  const RoutePlan p = route_plan(c);
  if (p.kind == RK_GEMV) {
    dim3 grid((unsigned)((c.E + 15) / 16), (unsigned)p.nsplit);
    hipLaunchKernelGGL(route_gemv_kernel, grid, dim3(kVWaves * 64), 0, s, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(w), (int)c.T, (int)c.H, (int)c.E, p.nsplit, part);
    return hipGetLastError();
  }
  if (p.kind == RK_GEMM) {
    if (c.E <= 32) return launch_route_gemm<1>(c, x, w, p.per, p.nsplit, part, s);
    if (c.E <= 64) return launch_route_gemm<2>(c, x, w, p.per, p.nsplit, part, s);
    if (c.E <= 128) return launch_route_gemm<4>(c, x, w, p.per, p.nsplit, part, s);
    return launch_route_gemm<8>(c, x, w, p.per, p.nsplit, part, s);
  }
  const int rbt = route_rbt(c.T, c.E);
  if (c.E <= 512)
    return rbt == 2 ? launch_route_wide<4, 2>(c, x, w, p.per, p.nsplit, part, s)
                    : launch_route_wide<4, 1>(c, x, w, p.per, p.nsplit, part, s);
  return launch_route_wide<8, 1>(c, x, w, p.per, p.nsplit, part, s);
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
