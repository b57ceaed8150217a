// Grouped expert GEMMs: gate/up with fused SwiGLU, then down (gfx950).
//
// Sources: niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", section
// "把一个大 FFN 换成一组小 FFN": each expert is a SwiGLU FFN (gate and up project
// H -> I, the SwiGLU activation joins them, down projects I -> H) and real
// implementations run the tokens of each expert as one batched ("grouped") GEMM;
// section "细粒度专家与共享专家": the shared expert sees every token.
//
// Work decomposition.  The dispatch step writes a device-side list of row chunks
// (expert group, first row, rows <= BM).  Workgroup p of the grid takes logical
// tile L(p) = (chunk, n-tile), with consecutive logical tiles placed on the same
// XCD (workgroups are dealt to the 8 XCDs round-robin), so the n-tiles of one
// chunk share its gathered token rows in that XCD's L2.  Workgroups past the
// device-side tile count exit at once, so the grid is sized on the host for the
// worst case and no host synchronisation is needed.
//
// bf16 tile: BM = 256 rows x BN = 128 weight rows x BK = 64, four waves in a
// 2 x 2 grid, each wave 128 x 64 of v_mfma_f32_32x32x16_bf16 (fp32 accumulators).
// Gate/up pass: the 128 weight rows are 64 gate rows and the same 64 up rows, and
// every wave owns 32 gate columns and the matching 32 up columns, so each lane
// holds gate and up of the same (row, i) and applies silu(g) * u in registers.
// The A tile is gathered straight from x through token_of_row (the gather of the
// dispatch step is fused into this loader) and both tiles are staged in LDS,
// double buffered, with 16-byte chunks XOR-swizzled by row to avoid bank
// conflicts on the MFMA operand reads.
#include <math.h>

#include "common.h"

namespace moe {
namespace {

constexpr int BM = kGemmBM;  // 256
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int A_LOADS = BM * BK / 8 / NT;  // 16-byte chunks per thread per K step (8)
constexpr int B_LOADS = BN * BK / 8 / NT;  // (4)

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

// Physical workgroup id -> logical tile id, XCD-contiguous; false past V.
__device__ __forceinline__ bool xcd_map(int p, int V, int& L) {
  if (p >= V) return false;
  const int xcd = p % kXcds, slot = p / kXcds;
  const int q = V / kXcds, r = V % kXcds;
  L = (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
  return true;
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ float silu_f(float g) { return g / (1.f + expf(-g)); }

template <int MODE>
__global__ __launch_bounds__(NT) void grouped_gemm_bf16(GemmArgs a, int n_tiles) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);          // [2][BM][BK]
  uint16_t* Bs = As + 2 * BM * BK;                           // [2][BN][BK]

  const int V = *a.n_chunks * n_tiles;
  int L;
  if (!xcd_map(blockIdx.x, V, L)) return;
  const int ci = L / n_tiles, nt = L % n_tiles;
  const Chunk ch = a.chunks[ci];
  const bool shared = ch.group == a.E;
  const int64_t K = a.K, N = a.N;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global source pointers (fixed for the whole K loop) ----
  const int lc = tid & 7;   // 16-byte chunk within the 64-wide K step
  const int lr = tid >> 3;  // first tile row of this thread (+32 per load)
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* ap[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int r = min(lr + 32 * i, ch.nrows - 1);
    const int64_t row = (int64_t)ch.row0 + r;
    int64_t src = row;
    if (a.gather != nullptr) src = shared ? row - a.shared_row0 : (int64_t)a.gather[row];
    ap[i] = A + src * K + lc * 8;
  }
  const uint16_t* bp[B_LOADS];
  if (MODE == MODE_GATEUP) {
    const uint16_t* Wg = static_cast<const uint16_t*>(shared ? a.ws0 : a.w0) +
                         (shared ? 0 : (int64_t)ch.group * N * K);
    const uint16_t* Wu = static_cast<const uint16_t*>(shared ? a.ws1 : a.w1) +
                         (shared ? 0 : (int64_t)ch.group * N * K);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int r = lr + 32 * i;  // 0..127: rows < 64 gate, >= 64 up
      const int64_t n = (int64_t)nt * 64 + (r & 63);
      bp[i] = (r < 64 ? Wg : Wu) + n * K + lc * 8;
    }
  } else {
    const uint16_t* Wd = static_cast<const uint16_t*>(shared ? a.ws0 : a.w0) +
                         (shared ? 0 : (int64_t)ch.group * N * K);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int64_t n = min((int64_t)nt * BN + lr + 32 * i, N - 1);
      bp[i] = Wd + n * K + lc * 8;
    }
  }
  int a_st[A_LOADS], b_st[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int r = lr + 32 * i;
    a_st[i] = r * BK + ((lc ^ (r & 7)) * 8);
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int r = lr + 32 * i;
    b_st[i] = r * BK + ((lc ^ (r & 7)) * 8);
  }

  // rows of this wave that hold real data (32-row blocks)
  const int wrow0 = wm * 128;
  const int nrb = max(0, min(4, (ch.nrows - wrow0 + 31) / 32));

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // B operand tile rows of this wave
  int brow[2];
  if (MODE == MODE_GATEUP) {
    brow[0] = wn * 32 + (lane & 31);       // gate
    brow[1] = 64 + wn * 32 + (lane & 31);  // up
  } else {
    brow[0] = wn * 64 + (lane & 31);
    brow[1] = wn * 64 + 32 + (lane & 31);
  }

  const int nk = (int)(K / BK);
  uint4 ra[A_LOADS], rb[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) ra[i] = ldg16(ap[i]);
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) rb[i] = ldg16(bp[i]);
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) *reinterpret_cast<uint4*>(As + a_st[i]) = ra[i];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) *reinterpret_cast<uint4*>(Bs + b_st[i]) = rb[i];
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t ko = (int64_t)(kt + 1) * BK;
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i) ra[i] = ldg16(ap[i] + ko);
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) rb[i] = ldg16(bp[i] + ko);
    }
    const uint16_t* Ab = As + (kt & 1) * BM * BK;
    const uint16_t* Bb = Bs + (kt & 1) * BN * BK;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int chunk = s * 2 + (lane >> 5);  // k = s*16 + (lane>>5)*8 .. +8
      bf16x8 bv[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = brow[j];
        bv[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Bb + r * BK + ((chunk ^ (r & 7)) * 8)));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < nrb) {
          const int r = wrow0 + i * 32 + (lane & 31);
          const bf16x8 av =
              __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Ab + r * BK + ((chunk ^ (r & 7)) * 8)));
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (more) {
      uint16_t* An = As + ((kt + 1) & 1) * BM * BK;
      uint16_t* Bn = Bs + ((kt + 1) & 1) * BN * BK;
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i) *reinterpret_cast<uint4*>(An + a_st[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) *reinterpret_cast<uint4*>(Bn + b_st[i]) = rb[i];
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds column (lane & 31), rows 8g + 4*(lane>>5) + r ----
  uint16_t* out = static_cast<uint16_t*>(a.out);
  const int col = lane & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= nrb) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wrow0 + i * 32 + 8 * g + 4 * (lane >> 5) + r;
        if (row >= ch.nrows) continue;
        const int64_t orow = (int64_t)ch.row0 + row;
        const int v = 4 * g + r;
        if (MODE == MODE_GATEUP) {
          const int64_t n = (int64_t)nt * 64 + wn * 32 + col;
          out[orow * N + n] = f32_to_bf16(silu_f(acc[i][0][v]) * acc[i][1][v]);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int64_t n = (int64_t)nt * BN + wn * 64 + j * 32 + col;
            if (n < N) out[orow * N + n] = f32_to_bf16(acc[i][j][v]);
          }
        }
      }
  }
}

// ---------------------------------------------------------------- fp32 path
// SIMT tiles of 64 rows: gate/up -> 32 output columns (32 gate + 32 up weight
// rows), down -> 64 output columns; 256 threads, 4 rows x (2+2 | 4) columns each.
constexpr int FBM = kGemmBMf32;  // 64
constexpr int FBK = 16;

template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32(GemmArgs a, int n_tiles) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][64 + 4];
  const int V = *a.n_chunks * n_tiles;
  int L;
  if (!xcd_map(blockIdx.x, V, L)) return;
  const int ci = L / n_tiles, nt = L % n_tiles;
  const Chunk ch = a.chunks[ci];
  const bool shared = ch.group == a.E;
  const int64_t K = a.K, N = a.N;
  const int tid = threadIdx.x;
  const float* A = static_cast<const float*>(a.A);

  // loader: 64 rows x 16 k = 1024 floats: thread -> row tid/4, 4 consecutive k
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int r_ld = min(lrow, ch.nrows - 1);
  const int64_t row_ld = (int64_t)ch.row0 + r_ld;
  int64_t src = row_ld;
  if (a.gather != nullptr) src = shared ? row_ld - a.shared_row0 : (int64_t)a.gather[row_ld];
  const float* ap = A + src * K + lk;
  const float* bp;
  if (MODE == MODE_GATEUP) {
    const float* W = static_cast<const float*>(lrow < 32 ? (shared ? a.ws0 : a.w0) : (shared ? a.ws1 : a.w1));
    const int64_t n = (int64_t)nt * 32 + (lrow & 31);
    bp = W + (shared ? 0 : (int64_t)ch.group * N * K) + n * K + lk;
  } else {
    const float* W = static_cast<const float*>(shared ? a.ws0 : a.w0);
    const int64_t n = min((int64_t)nt * 64 + lrow, N - 1);
    bp = W + (shared ? 0 : (int64_t)ch.group * N * K) + n * K + lk;
  }

  const int ty = tid >> 4, tx = tid & 15;  // rows ty*4.., columns by tx
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int64_t k0 = 0; k0 < K; k0 += FBK) {
    const float4 av = *reinterpret_cast<const float4*>(ap + k0);
    const float4 bv = *reinterpret_cast<const float4*>(bp + k0);
    As[lk + 0][lrow] = av.x; As[lk + 1][lrow] = av.y; As[lk + 2][lrow] = av.z; As[lk + 3][lrow] = av.w;
    Bs[lk + 0][lrow] = bv.x; Bs[lk + 1][lrow] = bv.y; Bs[lk + 2][lrow] = bv.z; Bs[lk + 3][lrow] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float ar[4], br[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = As[kk][ty * 4 + i];
      if (MODE == MODE_GATEUP) {
        br[0] = Bs[kk][tx * 2];      br[1] = Bs[kk][tx * 2 + 1];        // gate
        br[2] = Bs[kk][32 + tx * 2]; br[3] = Bs[kk][32 + tx * 2 + 1];   // up
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) br[j] = Bs[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* out = static_cast<float*>(a.out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= ch.nrows) continue;
    const int64_t orow = (int64_t)ch.row0 + row;
    if (MODE == MODE_GATEUP) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = (int64_t)nt * 32 + tx * 2 + j;
        out[orow * N + n] = silu_f(acc[i][j]) * acc[i][2 + j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = (int64_t)nt * 64 + tx * 4 + j;
        if (n < N) out[orow * N + n] = acc[i][j];
      }
    }
  }
}

template <int MODE>
hipError_t launch_gemm(const GemmArgs& a, int dtype, hipStream_t s) {
  if (dtype == MOE_BF16) {
    const int n_tiles = (int)(MODE == MODE_GATEUP ? a.N / 64 : (a.N + BN - 1) / BN);
    const int64_t grid = ((a.max_chunks * n_tiles + kXcds - 1) / kXcds) * kXcds;
    const size_t lds = (size_t)2 * (BM + BN) * BK * 2;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_bf16<MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(grouped_gemm_bf16<MODE>, dim3((unsigned)grid), dim3(NT), lds, s, a, n_tiles);
  } else {
    const int n_tiles = (int)(MODE == MODE_GATEUP ? a.N / 32 : (a.N + 63) / 64);
    const int64_t grid = ((a.max_chunks * n_tiles + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL(grouped_gemm_f32<MODE>, dim3((unsigned)grid), dim3(256), 0, s, a, n_tiles);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup(const GemmArgs& a, int dtype, hipStream_t s) { return launch_gemm<MODE_GATEUP>(a, dtype, s); }
hipError_t launch_down(const GemmArgs& a, int dtype, hipStream_t s) { return launch_gemm<MODE_DOWN>(a, dtype, s); }

}  // namespace moe
