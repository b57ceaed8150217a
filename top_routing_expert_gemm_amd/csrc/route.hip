// Router GEMM fused with the gate and the top-k selection (gfx950).
//
// Sources: niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", sections
// "把一个大 FFN 换成一组小 FFN" (router = one linear layer x @ W_router.T) and
// "路由器怎样选专家：top-k 与两种门控" (softmax / sigmoid gate, top-k,
// renormalisation, routed_scaling_factor); amazingdata.cn "moe-routing-hardest"
// (the routing steps).
//
// Kernels: the fused router of the stage entry point (route_bf16_kernel, below);
// for the layer, split-K partial logits that the select step (dispatch.hip) adds
// in slice order: route_gemm_kernel for batches above 16 tokens and E <= 256
// (128-token tiles, loader waves streaming the token rows, MFMA waves loading the
// router weights), route_gemv_kernel for batches of <= 16 tokens,
// route_partial_bf16_kernel for E > 256; route_f32_kernel for fp32.
//
// Fused bf16 path: one workgroup = 32 tokens x all E experts.  The 32 x 64 token tile is
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

// Large batches, E <= 256: one workgroup = 128 tokens x all experts over one
// slice of H.  128-token tiles take half the K slices that 256-token tiles
// would need to cover the chip, which halves the float32 partial logits
// written here and read back by the select step (at 8192 tokens, 256 experts:
// 34 MB in 4 slices instead of 67 MB in 8).
//
// Eight waves, two per SIMD, in two roles:
//   * four MFMA waves in a 2 x 2 grid (4 x 1 when the experts fit one 32-wide
//     block): a wave multiplies 64 tokens (two 32-row blocks) by half of the
//     32-expert blocks, so the tile's 128 x 32 NB accumulators live in their
//     registers.  They load the router weights (a few MB, served by L2)
//     straight to LDS, two K steps ahead, each wave load one 1 KB block of
//     eight rows with the swizzle applied on the source side.
//   * four loader waves stream the token rows (read once, from HBM) into
//     kLoadSets register sets, kLoadSets - 1 K steps ahead, and store each
//     step's rows to LDS one step before it is used.
// The token-row stream needs many bytes in flight per CU to run at HBM speed,
// and a wave's vector-memory counter completes in issue order: in one wave,
// each step's wait for its weights would also wait for every older token-row
// load.  Split over two kinds of waves, the weight waits of the MFMA waves
// leave the loader waves' deep queue alone.
// LDS: three buffers of token rows (16 KB) and of weights (32 NB KB), 128-byte
// rows, 16-byte chunks XOR-swizzled by row.  Each 64-wide step is four 16-wide
// substeps; the MFMA waves read the next substep's operands between the current
// substep's MFMAs (two operand register sets).  One barrier per step, which
// both roles reach: it sits before the last substep's MFMAs, when every MFMA
// wave has finished reading the step's buffers, and after the loader waves
// have stored the next step's rows.  Loads past the slice are clamped to its
// last step (issued, never used), so every step issues the same loads and
// every wait is an exact count.
typedef uint32_t rv4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void rlds_void;
constexpr int kGT = 128;                   // tokens per workgroup
constexpr int kGThreads = 512;             // four MFMA waves, then four loader waves
constexpr int kGNA = kGT * 8 / 256;        // token-row pieces per loader lane per step (4)
constexpr int kLoadSets = 6;               // loader register sets (token rows of 6 K steps)
constexpr int kRBufFlags = 0x00020000;     // raw buffer resource word 3 (gfx9 family)

__shared__ __attribute__((aligned(1024))) rv4 gA0[kGT * 8];
__shared__ __attribute__((aligned(1024))) rv4 gA1[kGT * 8];
__shared__ __attribute__((aligned(1024))) rv4 gA2[kGT * 8];
__shared__ __attribute__((aligned(1024))) rv4 gB0[256 * 8];
__shared__ __attribute__((aligned(1024))) rv4 gB1[256 * 8];
__shared__ __attribute__((aligned(1024))) rv4 gB2[256 * 8];
template <int U>
__device__ __forceinline__ rv4* g_a() {
  if constexpr (U == 0) return gA0;
  else if constexpr (U == 1) return gA1;
  else return gA2;
}
template <int U>
__device__ __forceinline__ rv4* g_b() {
  if constexpr (U == 0) return gB0;
  else if constexpr (U == 1) return gB1;
  else return gB2;
}

// Wave grid of a tile with NB 32-expert blocks: WT x WN MFMA waves, each RB
// token blocks of 32 rows x NBW expert blocks.
template <int NB>
struct RgShape {
  static constexpr int WN = NB >= 2 ? 2 : 1;
  static constexpr int WT = 4 / WN;
  static constexpr int RB = kGT / WT / 32;
  static constexpr int NBW = NB / WN;
  static_assert(WT * RB * 32 == kGT && WN * NBW == NB, "wave grid");
};

template <int NB>
struct RgOps {
  bf16x8 a[RgShape<NB>::RB];
  bf16x8 b[RgShape<NB>::NBW];
};

// Sized for the largest expert tile (entries a smaller tile does not use are
// never touched, so they cost no registers).
struct RgCtx {
  __amdgpu_buffer_rsrc_t rx;   // token rows of this tile (base: its first row)
  __amdgpu_buffer_rsrc_t rw;   // router weights
  uint32_t aoff[kGNA];         // loader lane: byte offset of token-row piece i at k = 0
  int aslot[kGNA];             // loader lane: LDS slot of token-row piece i
  uint32_t boff[8];            // MFMA lane: byte offset of this wave's weight block j at k = 0
  int ra[4], rb[4];            // MFMA lane: LDS slot of its first A / B operand row, per substep
  int wave;                    // wave index within its role
};

// Wait until at most N vector-memory loads of this wave are outstanding (the
// LDS and export counters are not waited on).
template <int N>
__device__ __forceinline__ void rg_wait_vm() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Wait for all but N vector-memory loads and for every LDS operation of this
// wave, then barrier.
template <int N>
__device__ __forceinline__ void rg_barrier() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- loader waves ----
__device__ __forceinline__ void rg_load_rows(rv4 (&r)[kGNA], const RgCtx& c, int kt) {
#pragma unroll
  for (int i = 0; i < kGNA; ++i) {
    r[i] = __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.aoff[i], kt * (kRBK * 2), 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}
template <int U>
__device__ __forceinline__ void rg_store_rows(const rv4 (&r)[kGNA], const RgCtx& c) {
#pragma unroll
  for (int i = 0; i < kGNA; ++i) g_a<U>()[c.aslot[i]] = r[i];
}
// Loader step R of the unrolled loop (relative step r = R mod kLoadSets): the
// rows of step r + 1 (set (R + 1) mod kLoadSets, complete once at most the
// (kLoadSets - 1) kGNA loads issued after them are outstanding) go to token
// buffer (r + 1) mod 3, which was last read in step r - 2; the set is refilled
// with step r + 1 + kLoadSets; barrier.
template <int R>
__device__ __forceinline__ void rg_loader_step(rv4 (&set)[kLoadSets][kGNA], const RgCtx& c, int t, int kl) {
  constexpr int J = (R + 1) % kLoadSets;
  rg_wait_vm<(kLoadSets - 1) * kGNA>();
  rg_store_rows<(R + 1) % 3>(set[J], c);
  __builtin_amdgcn_sched_barrier(0);
  rg_load_rows(set[J], c, min(t + 1 + kLoadSets, kl));
  rg_barrier<(kLoadSets - 1) * kGNA + kGNA>();
}
// The first n (< kLoadSets) loader steps of an unrolled group, for the steps left after the loop.
template <int R>
__device__ __forceinline__ void rg_loader_tail(rv4 (&set)[kLoadSets][kGNA], const RgCtx& c, int t, int kl, int n) {
  if constexpr (R < kLoadSets) {
    if (R < n) {
      rg_loader_step<R>(set, c, t + R, kl);
      rg_loader_tail<R + 1>(set, c, t, kl, n);
    }
  }
}

// ---- MFMA waves ----
template <int NB, int U>
__device__ __forceinline__ void rg_load_b(const RgCtx& c, int kt, int j) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rw, (rlds_void*)(g_b<U>() + (c.wave * NB + j) * 64), 16, c.boff[j],
                                           kt * (kRBK * 2), 0, 0);
}
// Operand q of substep s from buffers U: q < RB the token blocks, then the expert blocks.
template <int NB, int U>
__device__ __forceinline__ void rg_read(RgOps<NB>& o, const RgCtx& c, int s, int q) {
  constexpr int RB = RgShape<NB>::RB;
  if (q < RB) o.a[q] = __builtin_bit_cast(bf16x8, g_a<U>()[c.ra[s] + q * 256]);
  else o.b[q - RB] = __builtin_bit_cast(bf16x8, g_b<U>()[c.rb[s] + (q - RB) * 256]);
}

// Substep SS of the step in buffers U:
//   SS 0: weights of step t + 2 into weight buffer (U + 2) mod 3 (last read in
//         step t - 1), spread between the MFMAs;
//   SS 3: barrier (the weights of step t + 1 are in: only the NB loads of SS 0
//         may be outstanding; the loader waves have stored its token rows),
//         then the MFMAs with the first operand reads of step t + 1.
template <int NB, int U, int SS>
__device__ __forceinline__ void rg_substep(f32x16 (&acc)[RgShape<NB>::RB][RgShape<NB>::NBW], RgOps<NB> (&op)[2],
                                           const RgCtx& c, int t, int kl) {
  constexpr int RB = RgShape<NB>::RB;
  constexpr int NQ = RB + RgShape<NB>::NBW;          // operand reads per substep
  constexpr int NM = RB * RgShape<NB>::NBW;          // MFMAs per substep
  constexpr int NS = SS == 0 ? NB : 0;               // weight loads
  constexpr int RU = SS == 3 ? (U + 1) % 3 : U;      // buffers of the next substep's operands
  const int sn = (SS + 1) & 3;
  RgOps<NB>& cur = op[SS & 1];
  RgOps<NB>& nxt = op[(SS & 1) ^ 1];
  if constexpr (SS == 3) rg_barrier<NB>();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int n = m / RB, j = m % RB;
    acc[j][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[j], cur.b[n], acc[j][n], 0, 0, 0);
#pragma unroll
    for (int q = m * NS / NM; q < (m + 1) * NS / NM; ++q) {
      rg_load_b<NB, (U + 2) % 3>(c, min(t + 2, kl), q);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = m * NQ / NM; q < (m + 1) * NQ / NM; ++q) rg_read<NB, RU>(nxt, c, sn, q);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NB, int U>
__device__ __forceinline__ void rg_step(f32x16 (&acc)[RgShape<NB>::RB][RgShape<NB>::NBW], RgOps<NB> (&op)[2],
                                        const RgCtx& c, int t, int kl) {
  rg_substep<NB, U, 0>(acc, op, c, t, kl);
  rg_substep<NB, U, 1>(acc, op, c, t, kl);
  rg_substep<NB, U, 2>(acc, op, c, t, kl);
  rg_substep<NB, U, 3>(acc, op, c, t, kl);
}

template <int NB>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void route_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int H, int E, int steps_per_split,
    float* __restrict__ part) {
  static_assert(NB * 32 <= 256, "expert tile");
  using SH = RgShape<NB>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int t0 = blockIdx.x * kGT;
  const int ks = blockIdx.y;
  const int nk = H / kRBK;
  const int kb = ks * steps_per_split, ke = min(kb + steps_per_split, nk);
  const int kl = ke - 1;
  const int Epad = (E + 31) / 32 * 32;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);

  RgCtx c;
  c.wave = wid & 3;
  if (wid >= 4) {
    // loader wave l: pieces i = token rows 32 l + 8 i + lane / 8, logical chunk lane % 8
    c.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x + (int64_t)t0 * H), (short)0, -1, kRBufFlags);
#pragma unroll
    for (int i = 0; i < kGNA; ++i) {
      const int row = 32 * c.wave + 8 * i + (lane >> 3), ch = lane & 7;
      c.aoff[i] = (uint32_t)(((min(t0 + row, T - 1) - t0) * H + ch * 8) * 2);
      c.aslot[i] = row * 8 + (ch ^ rswz(row));
    }
    rv4 set[kLoadSets][kGNA];
#pragma unroll
    for (int s = 0; s < kLoadSets; ++s) rg_load_rows(set[s], c, min(kb + s, kl));
    rg_wait_vm<(kLoadSets - 1) * kGNA>();
    rg_store_rows<0>(set[0], c);
    __builtin_amdgcn_sched_barrier(0);
    rg_load_rows(set[0], c, min(kb + kLoadSets, kl));
    rg_barrier<kLoadSets * kGNA>();
    int t = kb;
    static_assert(kLoadSets == 6 && kLoadSets % 3 == 0, "the unrolled loop below");
    for (; t + 6 <= ke; t += 6) {
      rg_loader_step<0>(set, c, t, kl);
      rg_loader_step<1>(set, c, t + 1, kl);
      rg_loader_step<2>(set, c, t + 2, kl);
      rg_loader_step<3>(set, c, t + 3, kl);
      rg_loader_step<4>(set, c, t + 4, kl);
      rg_loader_step<5>(set, c, t + 5, kl);
    }
    rg_loader_tail<0>(set, c, t, kl, ke - t);
    rg_wait_vm<0>();
    return;
  }

  // MFMA wave (tw, ew): token rows tw * 32 RB .., expert blocks ew * NBW ..;
  // weight loads: wave load j fills rows 8 (wave NB + j) .. + 8; lane -> row +
  // lane / 8, physical slot lane % 8, loaded from the logical chunk that belongs there
  c.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w), (short)0, -1, kRBufFlags);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int r = 8 * (c.wave * NB + j) + (lane >> 3);
    const int ch = (lane & 7) ^ rswz(r);
    c.boff[j] = (uint32_t)((min(r, E - 1) * H + ch * 8) * 2);
  }
  const int tw = c.wave % SH::WT, ew = c.wave / SH::WT;
  const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    // lane -> row l32 of each 32-row block, logical chunk 4 h + s in substep s
    const int cs = (4 * h + s) ^ rswz(l32);
    c.ra[s] = (tw * SH::RB * 32 + l32) * 8 + cs;
    c.rb[s] = (ew * SH::NBW * 32 + l32) * 8 + cs;
  }

  f32x16 acc[SH::RB][SH::NBW];
#pragma unroll
  for (int j = 0; j < SH::RB; ++j)
#pragma unroll
    for (int m = 0; m < SH::NBW; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][m][v] = 0.f;

  RgOps<NB> op[2];
  // prologue: weights of steps kb and kb + 1 into buffers 0 and 1
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    rg_load_b<NB, 0>(c, kb, j);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    rg_load_b<NB, 1>(c, min(kb + 1, kl), j);
    __builtin_amdgcn_sched_barrier(0);
  }
  rg_barrier<NB>();
#pragma unroll
  for (int q = 0; q < SH::RB + SH::NBW; ++q) rg_read<NB, 0>(op[0], c, 0, q);

  int t = kb;
  for (; t + 3 <= ke; t += 3) {
    rg_step<NB, 0>(acc, op, c, t, kl);
    rg_step<NB, 1>(acc, op, c, t + 1, kl);
    rg_step<NB, 2>(acc, op, c, t + 2, kl);
  }
  if (t < ke) rg_step<NB, 0>(acc, op, c, t, kl);
  if (t + 1 < ke) rg_step<NB, 1>(acc, op, c, t + 1, kl);
  // the clamped weight loads of the last steps may still be writing LDS
  rg_wait_vm<0>();

  // lane holds expert column l32 of each block and token rows 8 g + 4 h + q.
  // Buffer stores over this slice's [T, Epad] partials: the resource's size
  // ends at row T, so the hardware drops the stores of rows past the batch.
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(part + (int64_t)ks * T * Epad, (short)0,
                                                                      T * Epad * 4, kRBufFlags);
#pragma unroll
  for (int j = 0; j < SH::RB; ++j)
#pragma unroll
    for (int m = 0; m < SH::NBW; ++m) {
      const int e0 = (ew * SH::NBW + m) * 32;
      if (e0 >= Epad) continue;  // the tile's blocks past E + padding
      const uint32_t o = (uint32_t)(((t0 + (tw * SH::RB + j) * 32 + 4 * h) * Epad + e0 + l32) * 4);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // the element is read into a scalar first: a bit cast of the vector-element expression itself
          // compiled to element 0 for every (g, q)
          const float v = acc[j][m][4 * g + q];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ro, o + (uint32_t)((8 * g + q) * Epad * 4), 0, 0);
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
    // one 128-token workgroup per CU in all, each slice at least four K steps long
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
