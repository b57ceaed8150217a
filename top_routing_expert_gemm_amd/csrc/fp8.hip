// FP8 expert weights for the decode path (gfx950).
//
// Source: niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", section
// "推理时：显存按总参数，计算按激活参数": the released DeepSeek-V3 weights are FP8,
// about one byte per parameter, and a small decode batch streams only the
// touched experts' weights.  Format (not given by the page): OCP E4M3 codes and
// one float32 scale per 128 x 128 block of each [out, in] weight matrix.
//
// * launch_quantize_fp8: one workgroup per 128 x 128 block.  scale = block
//   max |w| / 448 (1 for an all-zero block), float32; each weight becomes the
//   E4M3 code nearest to the float32 quotient w / scale, ties to the even code
//   (a software encoder with exactly that rounding; |w / scale| <= 448 up to
//   one rounding, saturated).
// * grouped_stream_fp8: the bf16 decode kernel's scheme with weights read as
//   bytes.  One wave owns NCG groups of 16 output columns of one chunk; each
//   128-wide K block of a code row is one 128-byte line, loaded whole
//   (non-temporal, eight lanes per row) and passed through the wave's own LDS
//   rows; from there a lane takes 32 code bytes of its operand row, converts
//   them exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and runs
//   four v_mfma_f32_16x16x32_bf16 into a block partial, which is added to the
//   result times the block's scale.  The token rows' fragments are loaded once
//   per block for all NCG groups.  Half the HBM bytes of bf16 weights per
//   token.
#include "common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- quantiser

__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (a >= 448.f) return sign | 0x7Eu;                                     // largest finite
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);            // m * 2^-9, m = 0..8
  int e;
  (void)frexpf(a, &e);                                                      // a in [2^(e-1), 2^e)
  const uint32_t m8 = (uint32_t)rintf(ldexpf(a, 4 - e));                  // 8 .. 16, ties to even
  const uint32_t code = ((uint32_t)(e + 6) << 3) + m8 - 8u;               // m8 = 16 carries into the exponent
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

template <typename T>
__device__ __forceinline__ float load_w(const T* p);
template <>
__device__ __forceinline__ float load_w<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}
template <>
__device__ __forceinline__ float load_w<float>(const float* p) {
  return *p;
}

// block (g, nb, kb): thread t covers row t / 2 of the block, columns 64 (t & 1) .. +64
template <typename T>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T* __restrict__ w, int64_t N, int64_t K,
                                                           uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float s_max[4];
  const int64_t nkb = K / kFp8Block, nnb = N / kFp8Block;
  const int64_t g = blockIdx.y;
  const int64_t nb = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = nb * kFp8Block + (tid >> 1);
  const int64_t col = kb * kFp8Block + (tid & 1) * 64;
  const T* src = w + (g * N + row) * K + col;
  float v[64];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    v[i] = load_w<T>(src + i);
    m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  if (lane == 0) s_max[wave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  if (tid == 0) scales[(g * nnb + nb) * nkb + kb] = scale;
  uint8_t* dst = codes + (g * N + row) * K + col;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t u[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) word |= e4m3_encode(v[16 * c + 4 * d + b] / scale) << (8 * b);
      u[d] = word;
    }
    reinterpret_cast<uint4*>(dst)[c] = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

// ------------------------------------------------------- streaming kernel

#ifndef MOE_FP8_FW
#define MOE_FP8_FW 4
#endif
#ifndef MOE_FP8_FP
#define MOE_FP8_FP 2
#endif
#ifndef MOE_FP8_NCG_GU
#define MOE_FP8_NCG_GU 1
#endif
#ifndef MOE_FP8_NCG_DN
#define MOE_FP8_NCG_DN 2
#endif
constexpr int FW = MOE_FP8_FW;  // waves per workgroup
constexpr int FP = MOE_FP8_FP;  // K blocks in flight per wave

// silu(g) = g / (1 + e^-g), with e^-g = 2^(-g log2 e) from the hardware base-2
// exponential and the quotient from the hardware reciprocal (each within about
// one ulp in fp32): five instructions per value instead of a correctly rounded
// exponential and division, in epilogues that apply it to every gate/up output.
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

// 8 codes (two dwords) -> 8 bf16, exact
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true);
  const uint4 u = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                             __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
  return __builtin_bit_cast(bf16x8, u);
}

// One wave: NCG groups of 16 output columns (16 NCG <= 128 consecutive columns,
// inside one 128-row scale block) of one chunk; the token rows' A fragments of
// each K block are loaded once and used for every group.
//
// Weight loads: a K block of a code row is one 128-byte line.  A large buffer
// read with the non-temporal hint streams at about 7.1 TB/s on this device
// (6.2-6.3 TB/s without), but only when each load instruction covers whole
// lines, which the MFMA operand layout does not.  So each lane loads one
// 16-byte piece of a whole line (eight lanes per row, eight rows per
// instruction), the block goes to the wave's own LDS rows (16-byte slots
// XOR-swizzled by row / 2: the stores and the operand reads of any 16 lanes
// fall on 64 distinct banks) and is read back in the operand layout; no
// barriers (the waves never share data).
__device__ __forceinline__ uint4 ld_nt(const uint8_t* p) {
  const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ int fp8_slot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <int MODE, int NCG>
__global__ __launch_bounds__(FW * 64) void grouped_stream_fp8(GemmArgs a, int n_wt) {
  constexpr bool GU = MODE == 0;  // gate/up pass (else down)
  constexpr int NM = GU ? 2 : 1;  // weight matrices per group
  static_assert(16 * NCG <= kFp8Block && kFp8Block % (16 * NCG) == 0, "column groups inside one scale block");
  __shared__ uint4 stage[FW][NM][NCG][16 * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int V = *a.n_chunks * n_wt;
  const int gw = blockIdx.x * FW + wave;
  if (gw >= V) return;  // whole wave; no barriers below
  const int ci = gw / n_wt, nt = gw % n_wt;
  const Chunk ch = a.chunks[ci];
  const bool shared = ch.group == a.E;
  const int64_t K = a.K, N = a.N;
  const int nkb = (int)(K / kFp8Block);
  const int r16 = lane & 15, g4 = lane >> 4;

  // A: token row r16 of the chunk (clamped); lane group g4 covers k = 32 g4 .. +32 of each block
  const int rc = min(r16, ch.nrows - 1);
  const int64_t row = (int64_t)ch.row0 + rc;
  int64_t src = row;
  if (a.gather != nullptr) src = shared ? row - a.shared_row0 : (int64_t)a.gather[row];
  const uint16_t* pa = static_cast<const uint16_t*>(a.A) + src * K + g4 * 32;
  // B: load (j, i) of a block takes code row n0 + 16 j + 8 i + (lane >> 3), 16-byte piece lane & 7
  const int brow = lane >> 3, bpc = lane & 7;
  const int64_t g = shared ? 0 : ch.group;
  const int64_t n0 = (int64_t)nt * 16 * NCG;
  const uint8_t* pb[NM];
  const float* qs[NM];
  const int64_t sbase = (g * (N / kFp8Block) + n0 / kFp8Block) * nkb;
  pb[0] = static_cast<const uint8_t*>(shared ? a.ws0 : a.w0) + (g * N + n0 + brow) * K + 16 * bpc;
  qs[0] = (shared ? a.ssc0 : a.sc0) + sbase;
  if constexpr (GU) {
    pb[1] = static_cast<const uint8_t*>(shared ? a.ws1 : a.w1) + (g * N + n0 + brow) * K + 16 * bpc;
    qs[1] = (shared ? a.ssc1 : a.sc1) + sbase;
  }

  f32x4 acc[NM][NCG];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int j = 0; j < NCG; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 ra[FP][4], rb[FP][NM][NCG][2];
  float sc[FP][NM];
  auto load = [&](int p, int kb) {
    const int64_t ko = (int64_t)kb * kFp8Block;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[p][i] = *reinterpret_cast<const uint4*>(pa + ko + 8 * i);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int j = 0; j < NCG; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) rb[p][m][j][i] = ld_nt(pb[m] + (int64_t)(16 * j + 8 * i) * K + ko);
      sc[p][m] = qs[m][kb];
    }
  };
  // store slots of this lane's two pieces, read slots of its two operand pieces (k = 32 g4 .. +32)
  const int ws0 = fp8_slot(brow, bpc), ws1 = fp8_slot(8 + brow, bpc);
  const int rs0 = fp8_slot(r16, 2 * g4), rs1 = fp8_slot(r16, 2 * g4 + 1);
  // One block: stage, read back, multiply; blocks past the end (K / 128 not a
  // multiple of FP) multiply a zero A operand.
  auto block = [&](int p, int kb) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int j = 0; j < NCG; ++j) {
        stage[wave][m][j][ws0] = rb[p][m][j][0];
        stage[wave][m][j][ws1] = rb[p][m][j][1];
      }
    const bool live = kb < nkb;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int j = 0; j < NCG; ++j) {
        const uint4 w[2] = {stage[wave][m][j][rs0], stage[wave][m][j][rs1]};
        f32x4 b = {0.f, 0.f, 0.f, 0.f};
        // substep s: lane group g4 supplies k = 32 g4 + 8 s .. +8 of this block, for A and B alike
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const uint4 wv = w[s2 >> 1];
          const bf16x8 bv = (s2 & 1) ? e4m3x8_to_bf16(wv.z, wv.w) : e4m3x8_to_bf16(wv.x, wv.y);
          const uint4 a4 = live ? ra[p][s2] : make_uint4(0u, 0u, 0u, 0u);
          b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a4), bv, b, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[m][j][q] = fmaf(sc[p][m], b[q], acc[m][j][q]);
      }
  };
  if (nkb > 0) {
    // FP blocks in flight, refilled unconditionally in the steady loop (exact
    // wait counts); the last round issues no loads.
    const int last = (nkb - 1) / FP * FP;
#pragma unroll
    for (int p = 0; p < FP; ++p) load(p, min(p, nkb - 1));
    for (int kb0 = 0; kb0 < last; kb0 += FP) {
#pragma unroll
      for (int p = 0; p < FP; ++p) {
        block(p, kb0 + p);
        load(p, min(kb0 + p + FP, nkb - 1));
      }
    }
#pragma unroll
    for (int p = 0; p < FP; ++p) block(p, last + p);
  }
  // lane holds output column n0 + 16 j + r16 for token rows 4 g4 + q
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rr = 4 * g4 + q;
    if (rr >= ch.nrows) continue;
    const int64_t orow = (int64_t)ch.row0 + rr;
#pragma unroll
    for (int j = 0; j < NCG; ++j) {
      const int64_t n = n0 + 16 * j + r16;
      if constexpr (GU)
        out[orow * N + n] = f32_to_bf16(silu_f(acc[0][j][q]) * acc[1][j][q]);
      else
        out[orow * N + n] = f32_to_bf16(acc[0][j][q]);
    }
  }
}

template <int MODE, int NCG>
hipError_t launch_fp8(const GemmArgs& a, hipStream_t s) {
  const int n_wt = (int)(a.N / (16 * NCG));
  const int64_t grid = (a.max_chunks * n_wt + FW - 1) / FW;
  hipLaunchKernelGGL((grouped_stream_fp8<MODE, NCG>), dim3((unsigned)grid), dim3(FW * 64), 0, s, a, n_wt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup_fp8(const GemmArgs& a, hipStream_t s) { return launch_fp8<0, MOE_FP8_NCG_GU>(a, s); }
hipError_t launch_down_fp8(const GemmArgs& a, hipStream_t s) { return launch_fp8<1, MOE_FP8_NCG_DN>(a, s); }

hipError_t launch_quantize_fp8(const void* w, int dtype, int64_t G, int64_t N, int64_t K, uint8_t* codes,
                               float* scales, hipStream_t s) {
  const dim3 grid((unsigned)((N / kFp8Block) * (K / kFp8Block)), (unsigned)G);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(quantize_fp8_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(w), N, K,
                       codes, scales);
  else
    hipLaunchKernelGGL(quantize_fp8_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(w), N, K, codes,
                       scales);
  return hipGetLastError();
}

}  // namespace moe
