// Grouped expert GEMMs: gate/up with fused SwiGLU, then down (gfx950).
//
// Sources: niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", section
// "把一个大 FFN 换成一组小 FFN": each expert is a SwiGLU FFN (gate and up project
// H -> I, the SwiGLU activation joins them, down projects I -> H) and real
// implementations run the tokens of each expert as one batched ("grouped") GEMM;
// section "细粒度专家与共享专家": the shared expert sees every token.
//
// Work decomposition.  The dispatch step writes device-side lists of row chunks
// (expert group, first row, rows <= the list's tile height).  Workgroup p of a
// launch takes logical tile L(p) = (chunk, n-tile), with consecutive logical
// tiles placed on the same XCD (workgroups are dealt to the 8 XCDs
// round-robin), so the n-tiles of one chunk share its gathered token rows in
// that XCD's L2.  Workgroups past the device-side tile count exit at once, so
// the grid is sized on the host for the worst case and no host synchronisation
// is needed.
//
// The kernels (launch_gemm picks one per pass and chunk list):
//   grouped_gemm_rs   256 x 256 tile, four waves, both operands register-staged
//                     two K steps ahead (bf16 prefill, the 256-row list);
//   grouped_gemm_ws   320 x 256 tile, eight waves, weights straight to LDS
//                     through three stages, token rows register-staged (bf16
//                     prefill, the 320-row list);
//   grouped_gemm_bf16 320 x 256 tile, eight waves, both operands straight to
//                     LDS (the 320-row list where the others' 32-bit offsets do
//                     not fit or K < 128);
//   grouped_gemm_wn   160 x 512 tile, eight waves, one persistent workgroup
//                     per CU (gate/up of lists whose chunks hold <= 160 rows);
//   grouped_stream_bf16  batches of <= 16 tokens: each wave streams 16 weight
//                     rows in whole 128-byte lines (non-temporal loads) and
//                     turns them into MFMA operands through its own LDS rows,
//                     no barriers (decode);
//   grouped_gemm_f32  fp32 SIMT tiles.
// In every bf16 tile kernel a wave owns matching gate and up columns in the
// gate/up pass, so each lane holds gate and up of the same (row, i) and applies
// silu(g) * u in registers; the A tile is gathered straight from x through
// token_of_row (the gather of the dispatch step is fused into the loader); the
// 16-byte chunks of each LDS row are XOR-swizzled by row so the MFMA operand
// reads are free of bank conflicts.
//
// 320-row direct-to-LDS tile: BM = 320 rows x BN = 256 weight rows, eight waves
// (two per SIMD) in a 2 x 4 grid, each wave up to 160 x 64 of
// v_mfma_f32_32x32x16_bf16 (fp32 accumulators).  A 320-row chunk holds a whole
// routed expert of the large workloads, so each expert's weights stream through
// one workgroup per n-tile.  Both tiles move global -> LDS with direct
// (global_load_lds_dwordx4) loads: A (token rows, from L2) in 64-wide K steps,
// whole 128-byte lines, through two stages, one step ahead; B (weights, from
// HBM) in 32-wide K steps through four stages, three steps ahead.
//
// Tile order: within one expert the chunks of an n-tile are adjacent (groups of
// up to four chunks), so a second row chunk of an expert reads the same weight
// tile right after the first, from L2.
#include <math.h>

#include "common.h"

namespace moe {
namespace {

constexpr int BM = kGemmBMdl;  // 320 rows: one chunk holds a whole routed expert of the large workloads
constexpr int BMW = BM / 2;    // rows per wave-row
constexpr int RB = BMW / 32;   // 32-row MFMA blocks per wave (5)
constexpr int BN = 256;
constexpr int NT = 512;
constexpr int NWAVES = NT / 64;
constexpr int SUPER = kChunkSuper;  // chunks of one group interleaved per n-tile
constexpr int BK = 32;         // K per step (and per B stage)
constexpr int B_BLK = BN / 16 / NWAVES;   // B blocks (16 rows x 64 B = 1 KB) per wave per stage (2)
constexpr int A_BLK = BM / 8 / NWAVES;    // A blocks (8 rows x 128 B = 1 KB) per wave per 64-wide A stage (5)
static_assert(A_BLK * 8 * NWAVES == BM && B_BLK * 16 * NWAVES == BN, "staging");
static_assert(2 * BM * 64 * 2 + 4 * BN * BK * 2 <= 160 * 1024, "LDS");

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// One LDS array per pipeline stage: distinct objects let the compiler tell the
// in-flight direct-to-LDS writes of one stage from the reads of another.
__shared__ __attribute__((aligned(1024))) uint16_t sA0[BM * 64];
__shared__ __attribute__((aligned(1024))) uint16_t sA1[BM * 64];
__shared__ __attribute__((aligned(1024))) uint16_t sB0[BN * BK];
__shared__ __attribute__((aligned(1024))) uint16_t sB1[BN * BK];
__shared__ __attribute__((aligned(1024))) uint16_t sB2[BN * BK];
__shared__ __attribute__((aligned(1024))) uint16_t sB3[BN * BK];

template <int S>
__device__ __forceinline__ uint16_t* stA() {
  if constexpr (S == 0) return sA0;
  else return sA1;
}
template <int S>
__device__ __forceinline__ uint16_t* stB() {
  if constexpr (S == 0) return sB0;
  else if constexpr (S == 1) return sB1;
  else if constexpr (S == 2) return sB2;
  else return sB3;
}

// XOR swizzles of the 16-byte chunks of a tile row: the 16 lanes of one
// ds_read_b128 cycle (rows r..r+15, one logical chunk) hit distinct banks on a
// 64-bank LDS, and the 8 lanes of a 32-bank cycle do too.
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }  // 4 chunks per 64-byte row
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }   // 8 chunks per 128-byte row

// Physical workgroup id -> logical tile id, XCD-contiguous; false past V.
__device__ __forceinline__ bool xcd_map(int p, int V, int& L) {
  if (p >= V) return false;
  const int xcd = p % kXcds, slot = p / kXcds;
  const int q = V / kXcds, r = V % kXcds;
  L = (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
  return true;
}

// Physical workgroup id -> logical tile id, dealing blocks of S consecutive
// logical tiles to the XCDs in turn (block b to XCD b % 8, each XCD taking its
// blocks in order); the tiles past the last whole round of 8 blocks are split
// into contiguous ranges as above.  With S = SUPER * n_tiles a block is one
// group of chunks that share weight tiles, so that sharing stays within one
// XCD's L2, while every XCD gets its share of each part of the list: the
// shared expert's chunks (last in a list, four to a weight tile, so lighter
// on HBM) spread over all XCDs instead of filling the last one or two.
__device__ __forceinline__ bool xcd_map_cyclic(int p, int V, int S, int& L) {
  if (p >= V) return false;
  const int Vm = V / (kXcds * S) * (kXcds * S);
  if (p < Vm) {
    const int x = p % kXcds, k = p / kXcds;
    L = ((k / S) * kXcds + x) * S + k % S;
    return true;
  }
  xcd_map(p - Vm, V - Vm, L);
  L += Vm;
  return true;
}

// Logical tile -> (chunk, n-tile): groups of up to SUPER chunks of one expert
// take the n-tiles in turn, so they share each weight tile.
__device__ __forceinline__ void tile_of(int L, int n_tiles, const Chunk* chunks, int& ci, int& nt) {
  const int c0 = L / n_tiles;
  const Chunk g = chunks[c0];
  const int sb = (c0 - g.gfirst) / SUPER;
  const int base = g.gfirst + sb * SUPER;
  const int cnt = min(SUPER, g.gcount - sb * SUPER);
  const int q = L - base * n_tiles;
  nt = q / cnt;
  ci = base + q % cnt;
}

// One 16-byte piece of an output row from the epilogue's LDS staging tile;
// `nt`: non-temporal store (the cache policy of data written once and read
// once later, by the next pass).
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_out(uint16_t* dst, const uint16_t* src, bool nt) {
  const v4u32 v = *reinterpret_cast<const v4u32*>(src);
  if (nt) __builtin_nontemporal_store(v, reinterpret_cast<v4u32*>(dst));
  else *reinterpret_cast<v4u32*>(dst) = v;
}

// silu(g) = g / (1 + e^-g), with e^-g = 2^(-g log2 e) from the hardware base-2
// exponential and the quotient from the hardware reciprocal (each within about
// one ulp in fp32): five instructions per value instead of a correctly rounded
// exponential and division, in epilogues that apply it to every gate/up output.
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// The value of the neighbouring lane (lane ^ 1): a DPP quad permutation
// [1, 0, 3, 2], one VALU move (no LDS round trip as a general shuffle takes).
__device__ __forceinline__ float lane_swap1(float v) {
  const int b = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false));
}

// Two floats to a pair of bf16 (round to nearest even), lo in bits 0..15: one
// v_cvt_pk_bf16_f32.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

// Wait until at most N of this wave's vector-memory loads are outstanding and
// its LDS reads are done, then barrier (no other fence: the stage buffers are
// the only shared state).  The wait is the s_waitcnt builtin (not inline asm) so
// the compiler's own wait-count tracking sees it and adds no wait of its own on
// the direct-to-LDS loads still in flight for other stages.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));  // vmcnt(N) expcnt(7) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct Frag {
  const uint16_t* ga[A_BLK];  // per-lane global source of each direct-to-LDS block
  const uint16_t* gb[B_BLK];
};

// A tile at (K offset 64 at) into A stage SA: block i of this wave holds rows
// (wave * A_BLK + i) * 8 .. + 8, whole 128-byte row pieces.
template <int SA>
__device__ __forceinline__ void issue_a(const Frag& f, int at, int wave) {
#pragma unroll
  for (int i = 0; i < A_BLK; ++i)
    __builtin_amdgcn_global_load_lds((glb_void*)(f.ga[i] + at * 64), (lds_void*)(stA<SA>() + (wave * A_BLK + i) * 512),
                                     16, 0, 0);
}
// B step kt (K offset 32 kt) into B stage SB: block i of this wave holds rows
// (wave * B_BLK + i) * 16 .. + 16, 64-byte row pieces.
template <int SB>
__device__ __forceinline__ void issue_b(const Frag& f, int kt, int wave) {
#pragma unroll
  for (int i = 0; i < B_BLK; ++i)
    __builtin_amdgcn_global_load_lds((glb_void*)(f.gb[i] + kt * BK), (lds_void*)(stB<SB>() + (wave * B_BLK + i) * 512),
                                     16, 0, 0);
}

// One 32-wide K step of this wave's NRB row blocks x two column blocks: A from
// half HALF of A stage SA (128-byte rows), B from B stage SB (64-byte rows).
template <int SA, int HALF, int SB, int NRB>
__device__ __forceinline__ void compute_step(f32x16 (&acc)[RB][2], int wrow0, const int (&brow)[2], int lane) {
  const uint16_t* Ab = stA<SA>();
  const uint16_t* Bb = stB<SB>();
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int cb = s * 2 + (lane >> 5);  // k = 16 s + 8 (lane >> 5) .. + 8 of the step
    const int ca = HALF * 4 + cb;
    bf16x8 bv[2], av[NRB];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = brow[j];
      bv[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Bb + r * BK + ((cb ^ swz4(r)) * 8)));
    }
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
      const int r = wrow0 + i * 32 + (lane & 31);
      av[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Ab + r * 64 + ((ca ^ swz8(r)) * 8)));
    }
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
  }
}

// K step kt (S = kt % 4: B stage S, A stage (S / 2) % 2, half S % 2).  Issue
// order per step: B step kt + 3 (B_BLK loads), then on even steps A tile
// kt / 2 + 1 (A_BLK loads), all clamped so every step issues the same.  Loads
// complete in issue order: at the barrier of an even step only B step kt + 2
// may be outstanding beyond what it needs (B step kt and A tile kt / 2); at an
// odd step B step kt was issued before one A tile, two B steps and another A
// tile.
template <int S, int NRB>
__device__ __forceinline__ void pipe_step(const Frag& f, f32x16 (&acc)[RB][2], int kt, int nk, int wrow0,
                                          const int (&brow)[2], int lane, int wave) {
  stage_barrier<(S % 2 == 0) ? B_BLK : 2 * B_BLK + 2 * A_BLK>();
  issue_b<(S + 3) % 4>(f, min(kt + 3, nk - 1), wave);
  if constexpr (S % 2 == 0) issue_a<((S / 2) + 1) % 2>(f, min(kt / 2 + 1, nk / 2 - 1), wave);
  if constexpr (NRB > 0) compute_step<(S / 2) % 2, S % 2, S, NRB>(acc, wrow0, brow, lane);
}

// The pipelined K loop of one wave computing NRB row blocks; nk (32-wide steps)
// is even, as K is a multiple of 64.  Every variant runs the same barriers and
// loads, so waves with different NRB stay in step.
template <int NRB>
__device__ __forceinline__ void k_loop(const Frag& f, f32x16 (&acc)[RB][2], int nk, int wrow0,
                                       const int (&brow)[2], int lane, int wave) {
  // the issues of steps -3, -2, -1: B 0; B 1, A 0; B 2
  issue_b<0>(f, 0, wave);
  issue_b<1>(f, min(1, nk - 1), wave);
  issue_a<0>(f, 0, wave);
  issue_b<2>(f, min(2, nk - 1), wave);
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) {  // no conditional memory traffic inside the loop
    pipe_step<0, NRB>(f, acc, kt, nk, wrow0, brow, lane, wave);
    pipe_step<1, NRB>(f, acc, kt + 1, nk, wrow0, brow, lane, wave);
    pipe_step<2, NRB>(f, acc, kt + 2, nk, wrow0, brow, lane, wave);
    pipe_step<3, NRB>(f, acc, kt + 3, nk, wrow0, brow, lane, wave);
  }
  if (kt < nk) {  // two steps left
    pipe_step<0, NRB>(f, acc, kt, nk, wrow0, brow, lane, wave);
    pipe_step<1, NRB>(f, acc, kt + 1, nk, wrow0, brow, lane, wave);
  }
  // the clamped refills of the last steps are still in flight: let them land
  // before the wave can retire
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
}

template <int MODE>
__global__ __launch_bounds__(NT) void grouped_gemm_bf16(GemmArgs a, int n_tiles) {
  const int V = *a.n_chunks * n_tiles;
  int L;
  if (!xcd_map_cyclic(blockIdx.x, V, SUPER * n_tiles, L)) return;
  int ci, nt;
  tile_of(L, n_tiles, a.chunks, ci, nt);
  const Chunk ch = a.chunks[ci];
  const bool shared = ch.group == a.E;
  const int64_t K = a.K, N = a.N;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;

  // ---- per-lane sources of the direct-to-LDS blocks ----
  // A block i of this wave holds tile rows (wave * A_BLK + i) * 8 .. + 8: lane ->
  // row lane / 8, physical chunk lane % 8, which holds logical chunk
  // (lane % 8) ^ swz8(row).  B block i: rows (wave * B_BLK + i) * 16 .. + 16, lane
  // -> row lane / 4, physical chunk lane % 4.  Rows past the chunk are clamped to
  // its last row (loaded, never used).
  Frag f;
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
#pragma unroll
  for (int i = 0; i < A_BLK; ++i) {
    const int r = (wave * A_BLK + i) * 8 + lane / 8;
    const int c = (lane % 8) ^ swz8(r);
    const int rc = min(r, ch.nrows - 1);
    const int64_t row = (int64_t)ch.row0 + rc;
    int64_t src = row;
    if (a.gather != nullptr) src = shared ? row - a.shared_row0 : (int64_t)a.gather[row];
    f.ga[i] = A + src * K + c * 8;
  }
  const int64_t goff = shared ? 0 : (int64_t)ch.group * N * K;
#pragma unroll
  for (int i = 0; i < B_BLK; ++i) {
    const int r = (wave * B_BLK + i) * 16 + lane / 4;
    const int c = (lane % 4) ^ swz4(r);
    const uint16_t* W;
    int64_t n;
    if (MODE == MODE_GATEUP) {  // rows < 128: gate, >= 128: up, same 128 columns of I
      W = static_cast<const uint16_t*>(r < 128 ? (shared ? a.ws0 : a.w0) : (shared ? a.ws1 : a.w1)) + goff;
      n = min((int64_t)nt * 128 + (r & 127), N - 1);
    } else {
      W = static_cast<const uint16_t*>(shared ? a.ws0 : a.w0) + goff;
      n = min((int64_t)nt * BN + r, N - 1);
    }
    f.gb[i] = W + n * K + c * 8;
  }

  // this wave's rows: wave-row wm covers tile rows wm*BMW .. +BMW; only the 32-row
  // blocks that hold data are computed (NRB is a template argument of the loop)
  const int wrow0 = wm * BMW;
  const int nrb = max(0, min(RB, (ch.nrows - wrow0 + 31) / 32));

  f32x16 acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  int brow[2];
  if (MODE == MODE_GATEUP) {
    brow[0] = wn * 32 + (lane & 31);        // gate
    brow[1] = 128 + wn * 32 + (lane & 31);  // up
  } else {
    brow[0] = wn * 64 + (lane & 31);
    brow[1] = wn * 64 + 32 + (lane & 31);
  }

  const int nk = (int)(K / BK);
  switch (nrb) {
    case 0: k_loop<0>(f, acc, nk, wrow0, brow, lane, wave); break;
    case 1: k_loop<1>(f, acc, nk, wrow0, brow, lane, wave); break;
    case 2: k_loop<2>(f, acc, nk, wrow0, brow, lane, wave); break;
    case 3: k_loop<3>(f, acc, nk, wrow0, brow, lane, wave); break;
    case 4: k_loop<4>(f, acc, nk, wrow0, brow, lane, wave); break;
    default: k_loop<5>(f, acc, nk, wrow0, brow, lane, wave); break;
  }
  static_assert(RB == 5, "k_loop dispatch");

  // ---- epilogue ----
  // Lane holds column (lane & 31) and rows 8g + 4*(lane>>5) + r of each 32x32
  // block.  The wave's output sub-tile goes through a wave-private LDS region
  // (its own stage buffer, free once every wave is past the K loop): lane pairs
  // swap one value so each lane writes two adjacent columns as one dword, then
  // rows leave as 16-byte stores.  Three row blocks per pass fit the smallest
  // stage buffer.
  __syncthreads();
  if (nrb > 0) {
    constexpr int NJ = MODE == MODE_GATEUP ? 1 : 2;  // 32-column output blocks of this wave
    constexpr int LDSR = NJ * 32 + 8;                // LDS row stride (elements), padded
    constexpr int PB = 3;                            // row blocks per pass
    static_assert(PB * 32 * LDSR * 2 <= BN * BK * 2 && BN * BK <= BM * 32, "epilogue pass fits a region");
    uint16_t* tile;
    switch (wave) {  // the two 40 KB A stages in halves, the four B stages
      case 0: tile = sA0; break;
      case 1: tile = sA0 + BM * 32; break;
      case 2: tile = sA1; break;
      case 3: tile = sA1 + BM * 32; break;
      case 4: tile = sB0; break;
      case 5: tile = sB1; break;
      case 6: tile = sB2; break;
      default: tile = sB3; break;
    }
    uint16_t* out = static_cast<uint16_t*>(a.out);
    const int64_t n0 = MODE == MODE_GATEUP ? (int64_t)nt * 128 + wn * 32 : (int64_t)nt * BN + wn * 64;
    const int col = lane & 31, h = lane >> 5;
    const bool odd = col & 1;
#pragma unroll
    for (int pass = 0; pass < RB; pass += PB) {
      if (pass >= nrb) break;
#pragma unroll
      for (int i = pass; i < pass + PB && i < RB; ++i) {
        if (i >= nrb) break;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int p = 0; p < 4; p += 2) {
              float va, vb;
              if (MODE == MODE_GATEUP) {
                va = silu_f(acc[i][0][4 * g + p]) * acc[i][1][4 * g + p];
                vb = silu_f(acc[i][0][4 * g + p + 1]) * acc[i][1][4 * g + p + 1];
              } else {
                va = acc[i][jj][4 * g + p];
                vb = acc[i][jj][4 * g + p + 1];
              }
              // even lane: (row ra, cols c, c+1); odd lane: (row ra+1, cols c-1, c)
              const float x = lane_swap1(odd ? va : vb);
              const int ra = (i - pass) * 32 + 8 * g + 4 * h + p;
              const uint32_t w = odd ? pack_bf16x2(x, vb) : pack_bf16x2(va, x);
              const int lr = odd ? ra + 1 : ra;
              const int lc = jj * 32 + (col & ~1);
              *reinterpret_cast<uint32_t*>(tile + lr * LDSR + lc) = w;
            }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
      const int nrows_pass = min(PB, nrb - pass) * 32;
      constexpr int CPRW = NJ * 4;  // 16-byte chunks per sub-tile row
      for (int idx = lane; idx < nrows_pass * CPRW; idx += kWave) {
        const int lr = idx / CPRW, c16 = idx % CPRW;
        const int row = wrow0 + pass * 32 + lr;
        const int64_t n = n0 + c16 * 8;
        if (row < ch.nrows && n < N)
          store_out(out + ((int64_t)ch.row0 + row) * N + n, tile + lr * LDSR + c16 * 8, a.nt_out);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next pass overwrites the region
    }
  }
}

// ------------------------------------------------ bf16 register-staged path
// A 256 x 256 tile with K steps of 64, four waves (one per SIMD: each wave has
// the SIMD's whole register file, 256 accumulators in AGPRs plus operands and
// staging).  Wave (wm, wn) computes 32-row blocks wm, wm + 2, ... (interleaved,
// so a short chunk spreads its MFMA work over all four SIMDs) against 128 tile
// columns, with v_mfma_f32_32x32x16_bf16.
//
// Data path: every lane fetches whole 128-byte row pieces (eight lanes per row,
// 16 bytes each) of the K tile after next into registers while the current
// tile is computed from LDS, then writes the next tile's registers into the
// other LDS buffer.  Two K tiles are thus in flight per workgroup, held in the
// register file rather than in LDS (two LDS buffers of 64 KB).  Loads are
// buffer loads (scalar base, 32-bit per-lane offsets); the weights, read once,
// with the non-temporal cache policy.  One barrier per K step.  The 16-byte
// chunks of each 128-byte LDS row are XOR-swizzled by row so the ds_write_b128
// stores and the MFMA operand reads are free of bank conflicts.
//
// Against the 320-row kernel: one wave per SIMD hides LDS waits and barriers
// less well, but the deeper weight prefetch and whole-line loads make a chunk
// cost about 0.88 of a 320-row chunk; the dispatch step sends an expert group
// to this tile when that is worth its smaller chunks (a layer runs both
// kernels, each over its own chunk list).
//
// Gate/up pass: the wave's four 32-column blocks are two gate blocks and the
// matching two up blocks (same I columns), so SwiGLU is applied in registers.
// A chunk's row count selects how many 32-row A blocks are fetched (NA) and how
// many row blocks each wave multiplies (NRB): both are template arguments, so
// the loop holds no conditional memory traffic and the compiler's wait counts
// are exact.
constexpr int RWMB = 4;            // 32-row blocks per wave
constexpr int RWNB = 4;            // 32-column blocks per wave
constexpr int RBM = 64 * RWMB;     // 256 tile rows
constexpr int RBN = 64 * RWNB;     // 256 tile columns (gate/up: 128 gate + 128 up)
constexpr int RBK = 64;            // K per step: 128-byte row pieces
constexpr int RNT = 256;           // threads
constexpr int RNAL = RBM / 32;     // A loads per lane per K step (at most)
constexpr int RNBL = RBN / 32;     // B loads per lane per K step
constexpr int RROWS = RBM + RBN;   // 128-byte LDS rows per buffer
static_assert(kGemmBMrs == RBM, "chunk lists are cut to the tile height");
static_assert(2 * RROWS * 128 <= 160 * 1024, "LDS");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct RsRegs {
  u32x4 a[RNAL];
  u32x4 b[RNBL];
};

// Buffer-resource loads: wave-uniform bases in scalar registers, one 32-bit
// per-lane offset per A row and one shared by all B rows, the K position and
// the B row group in the scalar offset.
struct RsSrc {
  __amdgpu_buffer_rsrc_t ra;   // A rows (x gathered, or the row space)
  __amdgpu_buffer_rsrc_t rg;   // gate (gate/up) or down weights of the tile's group
  __amdgpu_buffer_rsrc_t ru;   // up weights (gate/up)
  uint32_t aoff[RNAL];         // per-lane byte offset of A row piece i at k = 0
  uint32_t boff;               // per-lane byte offset of the row piece within a 32-row B group
  uint32_t bgrp[RNBL];         // byte offset of B group j within its matrix
};
constexpr int kBufFlags = 0x00020000;  // raw buffer resource word 3 (gfx9 family)
constexpr int kNonTemporal = 2;  // cache policy of the weight loads: each weight is read once

// Operand registers of one 16-wide substep.
struct RsOps {
  bf16x8 a[RWMB];
  bf16x8 b[RWNB];
};

// LDS barrier: this wave's LDS operations done, then workgroup barrier; global
// loads stay in flight.
__device__ __forceinline__ void rs_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Global load q of one K step (q < NA: A block q, else B block q - NA).
template <int MODE, int NA>
__device__ __forceinline__ void rs_load1(RsRegs& r, const RsSrc& s, int kt, int q) {
  const int ko = kt * (RBK * 2);
  if (q < NA) {
    r.a[q] = __builtin_amdgcn_raw_buffer_load_b128(s.ra, s.aoff[q], ko, 0);
  } else {
    const int j = q - NA;
    const bool up = MODE == MODE_GATEUP && (j & 3) >= 2;
    r.b[j] = __builtin_amdgcn_raw_buffer_load_b128(up ? s.ru : s.rg, s.boff, (int)s.bgrp[j] + ko, kNonTemporal);
  }
}

// LDS store q of one K step into buffer L; wr = this lane's uint4 slot within a
// 32-row group.
template <int NA>
__device__ __forceinline__ void rs_store1(const RsRegs& r, u32x4* L, int wr, int q) {
  if (q < NA) L[q * 256 + wr] = r.a[q];
  else L[(RNAL + q - NA) * 256 + wr] = r.b[q - NA];
}

// Operand read q of substep s from buffer L, in the order the MFMAs use them:
// A block 0, the RWNB B blocks, then A blocks 1 .. NRB-1.  ra[s] / rb[s]: this
// lane's uint4 slot of its first A / B operand row for substep s; A block a
// adds 2 x 32 rows, B block n adds 32 rows.
__device__ __forceinline__ void rs_read1(RsOps& o, const u32x4* L, const int (&ra)[4], const int (&rb)[4], int s,
                                         int q) {
  if (q == 0) o.a[0] = __builtin_bit_cast(bf16x8, L[ra[s]]);
  else if (q <= RWNB) o.b[q - 1] = __builtin_bit_cast(bf16x8, L[rb[s] + (q - 1) * 256]);
  else o.a[q - RWNB] = __builtin_bit_cast(bf16x8, L[ra[s] + (q - RWNB) * 512]);
}

// One 16-wide substep SS of K step t (in buffer S), with the memory traffic of
// the pipeline interleaved between its MFMAs (each kind spread over the
// substep in proportion, rs_side_table):
//   SS 0: the first half of the global loads of step t + 2 (register set S,
//         whose previous contents were stored in the step before), and the
//         operand reads of SS 1;
//   SS 1: the second half of those loads, and the operand reads of SS 2;
//   SS 2: the operand reads of SS 3, and the LDS stores of step t + 1 (register
//         set 1 - S into buffer 1 - S, whose last reads were before the
//         previous barrier);
//   SS 3: half the MFMAs, the barrier (step t + 1 is in LDS, step t's reads are
//         done), then the operand reads of SS 0 of step t + 1.
// Each group (side operations + one MFMA) is fenced with a scheduling barrier so
// the compiler keeps this order and only two operand sets are live.
// Order of the side operations of a substep with NL global loads, NR operand
// reads and NS LDS stores: the three sequences merged so each element comes
// when its share of the substep is due ((2i + 1) / 2n smallest first; reads win
// ties), computed at compile time.  kind: 0 global load, 1 operand read,
// 2 LDS store; idx: position within its sequence.
template <int N>
struct RsSideTable {
  int kind[N > 0 ? N : 1];
  int idx[N > 0 ? N : 1];
};
template <int NL, int NR, int NS>
constexpr RsSideTable<NL + NR + NS> rs_side_table() {
  RsSideTable<NL + NR + NS> t{};
  int il = 0, ir = 0, is = 0;
  for (int q = 0; q < NL + NR + NS; ++q) {
    // due times (2i + 1) / (2n) as cross-multiplied fractions; 4 / 1 = never
    const int64_t dl_n = il < NL ? 2 * il + 1 : 4, dl_d = il < NL ? 2 * NL : 1;
    const int64_t dr_n = ir < NR ? 2 * ir + 1 : 4, dr_d = ir < NR ? 2 * NR : 1;
    const int64_t ds_n = is < NS ? 2 * is + 1 : 4, ds_d = is < NS ? 2 * NS : 1;
    int k = 2;
    if (dr_n * dl_d <= dl_n * dr_d && dr_n * ds_d <= ds_n * dr_d) k = 1;
    else if (dl_n * ds_d <= ds_n * dl_d) k = 0;
    else k = 2;
    t.kind[q] = k;
    t.idx[q] = k == 0 ? il++ : (k == 1 ? ir++ : is++);
  }
  return t;
}

template <int MODE, int SS, int S, int NA, int NRB, bool LOAD, bool STORE, bool NEXT>
__device__ __forceinline__ void rs_substep(f32x16 (&acc)[RWMB][RWNB], RsRegs (&R)[2], RsOps (&op)[2],
                                           const RsSrc& src, u32x4* L0, u32x4* L1, int t, int wr,
                                           const int (&ra)[4], const int (&rb)[4]) {
  constexpr int M = NRB * RWNB;                  // MFMAs
  constexpr int NOP = NRB > 0 ? NRB + RWNB : 0;  // operand reads per substep
  constexpr int NLD = NA + RNBL;                 // global loads (and LDS stores) per K step
  constexpr int ld0 = SS == 0 ? 0 : NLD / 2;   // first global load of this substep
  constexpr int n_gl = !LOAD ? 0 : SS == 0 ? NLD / 2 : SS == 1 ? NLD - NLD / 2 : 0;
  constexpr int n_rd = SS < 3 ? NOP : (NEXT ? NOP : 0);
  constexpr int n_st = (SS == 2 && STORE) ? NLD : 0;
  constexpr bool BAR = SS == 3 && NEXT;
  constexpr int P = n_gl + n_rd + n_st;          // side operations (after the barrier in SS 3)
  constexpr int M0 = BAR ? M / 2 : 0;            // MFMAs before the barrier
  const u32x4* Lc = S == 0 ? L0 : L1;
  u32x4* Ln = S == 0 ? L1 : L0;
  const u32x4* Lr = SS < 3 ? Lc : Ln;            // buffer of the operands read here
  constexpr int sr = (SS + 1) & 3;               // substep they belong to
  RsOps& cur = op[SS & 1];
  RsOps& nxt = op[(SS & 1) ^ 1];

  // the three kinds of side operation, merged in proportion, so the operand
  // reads are spread over the substep instead of bunched
  constexpr RsSideTable<n_gl + n_rd + n_st> tab = rs_side_table<n_gl, n_rd, n_st>();
  auto side = [&](int q) {
    const int kind = tab.kind[q], idx = tab.idx[q];
    if (kind == 0) rs_load1<MODE, NA>(R[S], src, t + 2, ld0 + idx);
    else if (kind == 1) rs_read1(nxt, Lr, ra, rb, sr, idx);
    else rs_store1<NA>(R[1 - S], Ln, wr, idx);
  };
  auto mfma = [&](int m) {
    const int ai = m / RWNB, ni = m % RWNB;
    acc[ai][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[ai], cur.b[ni], acc[ai][ni], 0, 0, 0);
  };

#pragma unroll
  for (int m = 0; m < M0; ++m) {
    mfma(m);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (BAR) {
    rs_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr int MR = M - M0;  // MFMAs that carry the side operations
  if constexpr (MR == 0) {
#pragma unroll
    for (int q = 0; q < P; ++q) side(q);
    __builtin_amdgcn_sched_barrier(0);
  } else {
    constexpr int PPM = (P + MR - 1) / MR;  // side operations per MFMA, at most
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
      for (int j = 0; j < PPM; ++j) {  // constant trip count: fully unrolled, q is a constant
        const int q = m * P / MR + j;
        if (q < (m + 1) * P / MR) side(q);
      }
      mfma(M0 + m);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int MODE, int S, int NA, int NRB, bool LOAD, bool STORE, bool NEXT>
__device__ __forceinline__ void rs_step(f32x16 (&acc)[RWMB][RWNB], RsRegs (&R)[2], RsOps (&op)[2], const RsSrc& src,
                                        u32x4* L0, u32x4* L1, int t, int wr, const int (&ra)[4],
                                        const int (&rb)[4]) {
  rs_substep<MODE, 0, S, NA, NRB, LOAD, STORE, NEXT>(acc, R, op, src, L0, L1, t, wr, ra, rb);
  rs_substep<MODE, 1, S, NA, NRB, LOAD, STORE, NEXT>(acc, R, op, src, L0, L1, t, wr, ra, rb);
  rs_substep<MODE, 2, S, NA, NRB, LOAD, STORE, NEXT>(acc, R, op, src, L0, L1, t, wr, ra, rb);
  rs_substep<MODE, 3, S, NA, NRB, LOAD, STORE, NEXT>(acc, R, op, src, L0, L1, t, wr, ra, rb);
}

// The K loop: nk >= 2 steps, nk odd iff ODD (the tail is then one straight
// sequence, so no accumulator state merges across branches).
template <int MODE, int NA, int NRB, bool ODD>
__device__ __forceinline__ void rs_kloop(f32x16 (&acc)[RWMB][RWNB], const RsSrc& src, u32x4* L0, u32x4* L1, int nk,
                                         int wr, const int (&ra)[4], const int (&rb)[4]) {
  RsRegs R[2];
  RsOps op[2];
#pragma unroll
  for (int q = 0; q < NA + RNBL; ++q) rs_load1<MODE, NA>(R[0], src, 0, q);
#pragma unroll
  for (int q = 0; q < NA + RNBL; ++q) rs_load1<MODE, NA>(R[1], src, 1, q);
#pragma unroll
  for (int q = 0; q < NA + RNBL; ++q) rs_store1<NA>(R[0], L0, wr, q);
  rs_barrier();
  if constexpr (NRB > 0) {
#pragma unroll
    for (int q = 0; q < NRB + RWNB; ++q) rs_read1(op[0], L0, ra, rb, 0, q);
  }
  constexpr int TAIL = ODD ? 3 : 2;  // steps after the loop, the first in buffer 0
  int t = 0;
  for (; t + TAIL < nk; t += 2) {
    rs_step<MODE, 0, NA, NRB, true, true, true>(acc, R, op, src, L0, L1, t, wr, ra, rb);
    rs_step<MODE, 1, NA, NRB, true, true, true>(acc, R, op, src, L0, L1, t + 1, wr, ra, rb);
  }
  if constexpr (ODD) {
    rs_step<MODE, 0, NA, NRB, true, true, true>(acc, R, op, src, L0, L1, t, wr, ra, rb);
    rs_step<MODE, 1, NA, NRB, false, true, true>(acc, R, op, src, L0, L1, t + 1, wr, ra, rb);
    rs_step<MODE, 0, NA, NRB, false, false, false>(acc, R, op, src, L0, L1, t + 2, wr, ra, rb);
  } else {
    rs_step<MODE, 0, NA, NRB, false, true, true>(acc, R, op, src, L0, L1, t, wr, ra, rb);
    rs_step<MODE, 1, NA, NRB, false, false, false>(acc, R, op, src, L0, L1, t + 1, wr, ra, rb);
  }
}

// K loop and epilogue of one wave; NA A blocks are fetched for the workgroup,
// this wave multiplies NRB row blocks (tile rows (2a + wm) * 32 .. + 32).
template <int MODE, int NA, int NRB, bool ODD>
__device__ __forceinline__ void rs_wave(const GemmArgs& a, const Chunk& ch, int nt, const RsSrc& src, u32x4* L0,
                                        u32x4* L1, int wm, int wn, int lane, int wr) {
  const int64_t N = a.N;
  const int nk = (int)(a.K / RBK);
  int ra[4], rb[4];
  const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = (2 * s + h) ^ swz8(l32);
    ra[s] = (wm * 32 + l32) * 8 + c;
    rb[s] = (RBM + wn * 128 + l32) * 8 + c;
  }
  f32x16 acc[RWMB][RWNB];
#pragma unroll
  for (int i = 0; i < RWMB; ++i)
#pragma unroll
    for (int j = 0; j < RWNB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  rs_kloop<MODE, NA, NRB, ODD>(acc, src, L0, L1, nk, wr, ra, rb);

  // ---- epilogue ----
  // Lane holds column l32 and rows 8g + 4h + q (g, q < 4) of each 32 x 32 block.
  // Each row block goes through a wave-private LDS region (32 KB per wave, free
  // once every wave is past the K loop): lane pairs swap one value so each lane
  // writes two adjacent columns as one dword, then rows leave as 16-byte stores.
  rs_barrier();
  if constexpr (NRB > 0) {
    constexpr int NJ = MODE == MODE_GATEUP ? RWNB / 2 : RWNB;  // 32-column output blocks of this wave
    constexpr int LDSR = NJ * 32 + 8;                           // padded LDS row (elements)
    constexpr int CPRW = NJ * 4;                                // 16-byte chunks per output row
    static_assert(32 * LDSR * 2 <= 32 * 1024, "epilogue region");
    uint16_t* tile = reinterpret_cast<uint16_t*>(L0) + (wm + 2 * wn) * (32 * 1024 / 2);
    uint16_t* out = static_cast<uint16_t*>(a.out);
    const int64_t n0 = MODE == MODE_GATEUP ? (int64_t)nt * 128 + wn * 64 : (int64_t)nt * RBN + wn * 128;
    const bool odd = l32 & 1;
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int p = 0; p < 4; p += 2) {
            float va, vb;
            if (MODE == MODE_GATEUP) {
              va = silu_f(acc[i][jj][4 * g + p]) * acc[i][jj + 2][4 * g + p];
              vb = silu_f(acc[i][jj][4 * g + p + 1]) * acc[i][jj + 2][4 * g + p + 1];
            } else {
              va = acc[i][jj][4 * g + p];
              vb = acc[i][jj][4 * g + p + 1];
            }
            // even lane: (row ra, cols c, c+1); odd lane: (row ra+1, cols c-1, c)
            const float x = lane_swap1(odd ? va : vb);
            const int r = 8 * g + 4 * h + p;
            const uint32_t w = odd ? pack_bf16x2(x, vb) : pack_bf16x2(va, x);
            const int lr = odd ? r + 1 : r;
            *reinterpret_cast<uint32_t*>(tile + lr * LDSR + jj * 32 + (l32 & ~1)) = w;
          }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
      const int rowb = (2 * i + wm) * 32;
#pragma unroll
      for (int q = 0; q < 32 * CPRW / kWave; ++q) {
        const int idx = q * kWave + lane;
        const int lr = idx / CPRW, c16 = idx % CPRW;
        const int row = rowb + lr;
        const int64_t n = n0 + c16 * 8;
        if (row < ch.nrows && n < N)
          store_out(out + ((int64_t)ch.row0 + row) * N + n, tile + lr * LDSR + c16 * 8, a.nt_out);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next block overwrites the region
    }
  }
}

template <int MODE, int NA, bool ODD>
__device__ __forceinline__ void rs_run(const GemmArgs& a, const Chunk& ch, int nt, u32x4* L0, u32x4* L1) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const bool shared = ch.group == a.E;
  const int64_t K = a.K, N = a.N;

  // loader: lane -> row (tid / 8) of each 32-row group, logical 16-byte chunk tid % 8
  const int lrow = tid >> 3, lchunk = tid & 7;
  const int wr = lrow * 8 + (lchunk ^ swz8(lrow));
  RsSrc src;
  src.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.A), (short)0, -1, kBufFlags);
#pragma unroll
  for (int i = 0; i < RNAL; ++i) {
    const int rc = min(i * 32 + lrow, ch.nrows - 1);
    const int64_t row = (int64_t)ch.row0 + rc;
    int64_t sr = row;
    if (a.gather != nullptr) sr = shared ? row - a.shared_row0 : (int64_t)a.gather[row];
    src.aoff[i] = (uint32_t)((sr * K + lchunk * 8) * 2);  // A spans < 4 GiB (checked by the host)
  }
  const int64_t goff = shared ? 0 : (int64_t)ch.group * N * K;
  const uint16_t* Wg = static_cast<const uint16_t*>(shared ? a.ws0 : a.w0) + goff;
  const uint16_t* Wu = MODE == MODE_GATEUP ? static_cast<const uint16_t*>(shared ? a.ws1 : a.w1) + goff : Wg;
  src.rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Wg), (short)0, -1, kBufFlags);
  src.ru = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Wu), (short)0, -1, kBufFlags);
#pragma unroll
  for (int j = 0; j < RNBL; ++j) {
    // B tile rows 32 j .. 32 j + 31; rows of wave column wn are [128 wn, 128 wn + 128)
    int64_t n;
    if (MODE == MODE_GATEUP)  // per wave column: 64 gate rows, then the same 64 up rows
      n = (int64_t)nt * 128 + (j >> 2) * 64 + (j & 1) * 32;
    else
      n = (int64_t)nt * RBN + j * 32;
    // a group past N is clamped to the last 32 rows (loaded, never stored); N is a multiple of 32
    src.bgrp[j] = (uint32_t)(min(n, N - 32) * K * 2);
  }
  src.boff = (uint32_t)((lrow * K + lchunk * 8) * 2);

  if (wm == 0) rs_wave<MODE, NA, (NA + 1) / 2, ODD>(a, ch, nt, src, L0, L1, wm, wn, lane, wr);
  else rs_wave<MODE, NA, NA / 2, ODD>(a, ch, nt, src, L0, L1, wm, wn, lane, wr);
}

template <int MODE, bool ODD>
__global__ __launch_bounds__(RNT) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_rs(GemmArgs a, int n_tiles) {
  __shared__ __attribute__((aligned(1024))) u32x4 lds[2 * RROWS * 8];
  const int V = *a.n_chunks * n_tiles;
  int L;
  if (!xcd_map_cyclic(blockIdx.x, V, SUPER * n_tiles, L)) return;
  int ci, nt;
  tile_of(L, n_tiles, a.chunks, ci, nt);
  const Chunk ch = a.chunks[ci];
  u32x4* L0 = lds;
  u32x4* L1 = lds + RROWS * 8;
  switch ((ch.nrows + 31) / 32) {
    case 1: rs_run<MODE, 1, ODD>(a, ch, nt, L0, L1); break;
    case 2: rs_run<MODE, 2, ODD>(a, ch, nt, L0, L1); break;
    case 3: rs_run<MODE, 3, ODD>(a, ch, nt, L0, L1); break;
    case 4: rs_run<MODE, 4, ODD>(a, ch, nt, L0, L1); break;
    case 5: rs_run<MODE, 5, ODD>(a, ch, nt, L0, L1); break;
    case 6: rs_run<MODE, 6, ODD>(a, ch, nt, L0, L1); break;
    case 7: rs_run<MODE, 7, ODD>(a, ch, nt, L0, L1); break;
    default: rs_run<MODE, 8, ODD>(a, ch, nt, L0, L1); break;
  }
  static_assert(RNAL == 8, "row-block dispatch");
}

// The register-staged kernel takes a pass when it has at least two K steps and
// its 32-bit buffer offsets cover A and one expert's weights (the chunk height
// of the layer already says so; a pass it does not fit runs on the
// direct-to-LDS kernel, which takes chunks of up to 320 rows).
bool rs_fits(const GemmArgs& a) {
  const int64_t lim = int64_t(1) << 32;
  return a.K >= 2 * RBK && a.a_rows * a.K * 2 < lim && a.N * a.K * 2 < lim;
}

// ------------------------------------ bf16 register-staged path, 320-row tile
// The 320 x 256 tile of the direct-to-LDS kernel with whole-line loads of both
// operands: eight waves (two per SIMD) in a 2 x 4 grid, wave (wm, wn) computing
// the interleaved 32-row blocks 2a + wm (a < 5) against 64 tile columns
// (gate/up: 32 gate columns and the same 32 up columns), 160 accumulators per
// lane.
//
// Every load is a whole 128-byte row piece (K steps of 64), for both operands:
// a CU's loads are limited by the requests it has in flight more than by
// bytes, and a step that fetches its weight rows as whole lines instead of
// 64-byte halves moves the same bytes about 18% faster.  The weights go
// straight to LDS (buffer_load ... lds, chunks swizzled on the source side)
// through three 32 KB stages, issued two K steps ahead; the token rows (from
// L2) go through registers, issued one step ahead, into one 40 KB buffer (the
// faster path for L2 hits, and what leaves LDS room for the third weight
// stage).  Two barriers per step: before the token rows of step t + 1
// overwrite those of step t (every wave done reading them), and after (step
// t + 1 complete in LDS).  Waves w and w + 4 share a SIMD and take the two row
// halves, so a chunk of 9 row blocks keeps every SIMD equally busy.  Within a
// 16-wide substep the MFMAs run column-major
// (every row block against B column block 0, then against block 1), so the
// next substep's operands are read into the registers the current ones free:
// B block 0 half-way through, each A block after its last use, B block 1 at
// the end.
constexpr int WNT = 512;           // eight waves, two per SIMD
constexpr int WRB = 5;             // 32-row blocks per wave (at most)
constexpr int WNB = 2;             // 32-column blocks per wave
// Tile shapes: V = 0 is the 320 x 256 tile (2 x 4 waves, three weight stages
// issued two K steps ahead); V = 1 is a 160 x 512 tile (1 x 8 waves, two 64 KB
// weight stages issued one step ahead) for lists whose chunks all hold at most
// 160 rows (capacity-limited layers): such a chunk fills only half of a
// 320-row tile, and twice the columns halve the token-row bytes fetched per
// weight byte.
template <int V>
struct Ws {
  static constexpr int WM = V == 0 ? 2 : 1;      // wave rows
  static constexpr int WN = 8 / WM;              // wave columns
  static constexpr int ST = V == 0 ? 3 : 2;      // weight stages
  static constexpr int BM = 32 * WRB * WM;       // 320 / 160 tile rows
  static constexpr int BN = 32 * WNB * WN;       // 256 / 512 tile columns
  static constexpr int AL = (BM + 63) / 64;      // 64-row A groups (loads per lane per K step, at most)
  static constexpr int BL = BN / 64;             // 64-row B groups (loads per lane per K step)
  static constexpr int AS = WM * 256;            // LDS distance (16-byte slots) between a wave's row blocks
  static_assert(AL * 64 * 128 + ST * BN * 128 <= 160 * 1024, "LDS");
  static_assert(WM * WN * 64 == WNT, "eight waves");
};
constexpr int WBM = Ws<0>::BM;
constexpr int kWideRows = Ws<1>::BM;
static_assert(kGemmBMdl == WBM && kGemmBMwn == kWideRows, "chunk lists are cut to the tile height");

// Distinct objects, so the compiler can tell the direct writes in flight to
// one stage from the reads of another.
__shared__ __attribute__((aligned(1024))) u32x4 sWA[Ws<0>::AL * 512];
__shared__ __attribute__((aligned(1024))) u32x4 sWB0[Ws<0>::BL * 512];
__shared__ __attribute__((aligned(1024))) u32x4 sWB1[Ws<0>::BL * 512];
__shared__ __attribute__((aligned(1024))) u32x4 sWB2[Ws<0>::BL * 512];
__shared__ __attribute__((aligned(1024))) u32x4 sVA[Ws<1>::AL * 512];
__shared__ __attribute__((aligned(1024))) u32x4 sVB0[Ws<1>::BL * 512];
__shared__ __attribute__((aligned(1024))) u32x4 sVB1[Ws<1>::BL * 512];
template <int V>
__device__ __forceinline__ u32x4* wsA() {
  if constexpr (V == 0) return sWA;
  else return sVA;
}
template <int V, int B>
__device__ __forceinline__ u32x4* wsB() {
  if constexpr (V == 0) {
    if constexpr (B == 0) return sWB0;
    else if constexpr (B == 1) return sWB1;
    else return sWB2;
  } else {
    if constexpr (B == 0) return sVB0;
    else return sVB1;
  }
}

// Sized for both tile shapes (the unused entries of the smaller one are never
// touched, so they cost no registers).
constexpr int kWsMaxAL = Ws<0>::AL > Ws<1>::AL ? Ws<0>::AL : Ws<1>::AL;
constexpr int kWsMaxBL = Ws<0>::BL > Ws<1>::BL ? Ws<0>::BL : Ws<1>::BL;
struct WsRegs {
  u32x4 a[kWsMaxAL];
};

struct WsSrc {
  __amdgpu_buffer_rsrc_t ra;   // A rows
  __amdgpu_buffer_rsrc_t rb;   // this wave's weight matrix (gate/up: gate for waves 0-3, up for 4-7)
  uint32_t aoff[kWsMaxAL];     // per-lane byte offset of A piece i at k = 0
  uint32_t boff;               // per-lane byte offset of the (source-swizzled) piece within a B row group
  uint32_t bgrp[kWsMaxBL];     // byte offset of B row group j within the matrix
  int wave;
};

struct WsOps {
  bf16x8 a[WRB];
  bf16x8 b[WNB];
};

// Token rows of A group i (tile rows 64 i + lane row) of K step kt into registers.
template <int V>
__device__ __forceinline__ void ws_load_a(WsRegs& r, const WsSrc& s, int kt, int i) {
  r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(s.ra, s.aoff[i], kt * (RBK * 2), 0);
}
// Weights of B row group j of K step kt straight into stage B (rows 64 j +
// 8 wave .. + 8: one 1 KB block per wave).
template <int V, int B>
__device__ __forceinline__ void ws_load_b(const WsSrc& s, int kt, int j) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rb, (lds_void*)(wsB<V, B>() + j * 512 + s.wave * 64), 16, s.boff,
                                           (int)s.bgrp[j] + kt * (RBK * 2), 0, kNonTemporal);
}

// One 16-wide substep SS of K step t, reading weight stage BS (ST stages):
//   SS 0, first half (MFMAs (a, 0) for every row block a): the loads of the
//         token rows of step t + 1 (LA) and then of the weights of step
//         t + ST - 1 into stage (BS + ST - 1) % ST, the stage step t - 1 used
//         (LB), each fenced so the issue order holds;
//   SS 3 (NEXT): the first barrier (every wave is done reading step t's token
//         rows: its last reads were in SS 2), then the first half carrying the
//         stores of step t + 1's token rows, then the second barrier, after
//         waiting for all of this wave's loads but the weights of step t + 2
//         (three stages: issued last): step t + 1 is complete in LDS;
//   then B block 0 of the next substep (step t + 1's stage in SS 3), and the
//   second half, MFMAs (a, 1), each followed by the read of the next
//   substep's A block a; last, B block 1 of the next substep.
template <int V, int MODE, int SS, int BS, int NAL, int NRB, bool LA, bool LB, bool NEXT>
__device__ __forceinline__ void ws_substep(f32x16 (&acc)[WRB][WNB], WsRegs& R, WsOps (&op)[2],
                                           const WsSrc& src, int t, int wr, const int (&ra)[4],
                                           const int (&rb)[4]) {
  using S = Ws<V>;
  constexpr int NA0 = (SS == 0 && LA) ? NAL : 0;
  constexpr int P = SS == 0 ? NA0 + (LB ? S::BL : 0) : ((SS == 3 && NEXT) ? NAL : 0);  // first-half side operations
  constexpr bool RD = SS < 3 || NEXT;  // operands of the next substep are read here
  const u32x4* Lb = wsB<V, SS < 3 ? BS : (BS + 1) % S::ST>();
  u32x4* La = wsA<V>();
  constexpr int sr = (SS + 1) & 3;
  constexpr int BN_ = (BS + S::ST - 1) % S::ST;  // stage of the weights loaded here
  WsOps& cur = op[SS & 1];
  WsOps& nxt = op[(SS & 1) ^ 1];
  auto side = [&](int q) {
    if constexpr (SS == 0) {
      if (q < NA0) ws_load_a<V>(R, src, t + 1, q);
      else ws_load_b<V, BN_>(src, t + Ws<V>::ST - 1, q - NA0);
    } else {
      La[q * 512 + wr] = R.a[q];
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (SS == 3 && NEXT) {
    rs_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (NRB == 0) {
#pragma unroll
    for (int q = 0; q < P; ++q) side(q);
  } else {
    constexpr int PPM = (P + NRB - 1) / NRB;
#pragma unroll
    for (int m = 0; m < NRB; ++m) {
#pragma unroll
      for (int j = 0; j < PPM; ++j) {
        const int q = m * P / NRB + j;
        if (q < (m + 1) * P / NRB) side(q);
      }
      acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[m], cur.b[0], acc[m][0], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (SS == 3 && NEXT) {
    stage_barrier<(LB && S::ST == 3) ? S::BL : 0>();
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (RD && NRB > 0) nxt.b[0] = __builtin_bit_cast(bf16x8, Lb[rb[sr]]);
#pragma unroll
  for (int m = 0; m < NRB; ++m) {
    acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[m], cur.b[1], acc[m][1], 0, 0, 0);
    if constexpr (RD) nxt.a[m] = __builtin_bit_cast(bf16x8, La[ra[sr] + m * S::AS]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (RD && NRB > 0) nxt.b[1] = __builtin_bit_cast(bf16x8, Lb[rb[sr] + 256]);
  __builtin_amdgcn_sched_barrier(0);
}

template <int V, int MODE, int BS, int NAL, int NRB, bool LA, bool LB, bool NEXT>
__device__ __forceinline__ void ws_step(f32x16 (&acc)[WRB][WNB], WsRegs& R, WsOps (&op)[2], const WsSrc& src,
                                        int t, int wr, const int (&ra)[4], const int (&rb)[4]) {
  ws_substep<V, MODE, 0, BS, NAL, NRB, LA, LB, NEXT>(acc, R, op, src, t, wr, ra, rb);
  ws_substep<V, MODE, 1, BS, NAL, NRB, LA, LB, NEXT>(acc, R, op, src, t, wr, ra, rb);
  ws_substep<V, MODE, 2, BS, NAL, NRB, LA, LB, NEXT>(acc, R, op, src, t, wr, ra, rb);
  ws_substep<V, MODE, 3, BS, NAL, NRB, LA, LB, NEXT>(acc, R, op, src, t, wr, ra, rb);
}

// The K loop over nk >= 2 steps.  Three weight stages, R = (nk - 2) % 3: steps
// 0 .. nk - 3 load both operands ahead (the loop, unrolled by the three
// stages, then R more), step nk - 2 loads only the token rows of the last
// step, step nk - 1 nothing.  Two stages, R = (nk - 1) % 2: steps 0 .. nk - 2
// load both operands of the next step (the loop unrolled by two, then R more),
// step nk - 1 nothing.  Step t reads weight stage t % ST.
template <int V, int MODE, int NAL, int NRB, int R>
__device__ __forceinline__ void ws_kloop(f32x16 (&acc)[WRB][WNB], const WsSrc& src, int nk, int wr,
                                         const int (&ra)[4], const int (&rb)[4]) {
  using S = Ws<V>;
  WsRegs Rg;
  WsOps op[2];
  u32x4* La = wsA<V>();
#pragma unroll
  for (int i = 0; i < NAL; ++i) {
    ws_load_a<V>(Rg, src, 0, i);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < S::BL; ++j) {
    ws_load_b<V, 0>(src, 0, j);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (S::ST == 3) {
#pragma unroll
    for (int j = 0; j < S::BL; ++j) {
      ws_load_b<V, 1>(src, 1, j);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < NAL; ++i) La[i * 512 + wr] = Rg.a[i];
  // token rows and weights of step 0 in LDS (three stages: step 1's weights may be in flight)
  stage_barrier<S::ST == 3 ? S::BL : 0>();
  if constexpr (NRB > 0) {
    const u32x4* L0 = wsB<V, 0>();
    op[0].b[0] = __builtin_bit_cast(bf16x8, L0[rb[0]]);
#pragma unroll
    for (int m = 0; m < NRB; ++m) op[0].a[m] = __builtin_bit_cast(bf16x8, La[ra[0] + m * S::AS]);
    op[0].b[1] = __builtin_bit_cast(bf16x8, L0[rb[0] + 256]);
  }
  int t = 0;
  if constexpr (S::ST == 3) {
    for (; t + 3 <= nk - 2; t += 3) {
      ws_step<V, MODE, 0, NAL, NRB, true, true, true>(acc, Rg, op, src, t, wr, ra, rb);
      ws_step<V, MODE, 1, NAL, NRB, true, true, true>(acc, Rg, op, src, t + 1, wr, ra, rb);
      ws_step<V, MODE, 2, NAL, NRB, true, true, true>(acc, Rg, op, src, t + 2, wr, ra, rb);
    }
    if constexpr (R >= 1) ws_step<V, MODE, 0, NAL, NRB, true, true, true>(acc, Rg, op, src, t, wr, ra, rb);
    if constexpr (R >= 2) ws_step<V, MODE, 1, NAL, NRB, true, true, true>(acc, Rg, op, src, t + 1, wr, ra, rb);
    ws_step<V, MODE, R % 3, NAL, NRB, true, false, true>(acc, Rg, op, src, t + R, wr, ra, rb);
    ws_step<V, MODE, (R + 1) % 3, NAL, NRB, false, false, false>(acc, Rg, op, src, t + R + 1, wr, ra, rb);
  } else {
    for (; t + 2 <= nk - 1; t += 2) {
      ws_step<V, MODE, 0, NAL, NRB, true, true, true>(acc, Rg, op, src, t, wr, ra, rb);
      ws_step<V, MODE, 1, NAL, NRB, true, true, true>(acc, Rg, op, src, t + 1, wr, ra, rb);
    }
    if constexpr (R >= 1) ws_step<V, MODE, 0, NAL, NRB, true, true, true>(acc, Rg, op, src, t, wr, ra, rb);
    ws_step<V, MODE, R % 2, NAL, NRB, false, false, false>(acc, Rg, op, src, t + R, wr, ra, rb);
  }
}

// K loop and epilogue of one wave, which multiplies NRB row blocks (tile rows
// (WM a + wm) * 32 .. + 32); NAL 64-row A groups are fetched for the workgroup.
template <int V, int MODE, int NAL, int NRB, int R>
__device__ __forceinline__ void ws_wave(const GemmArgs& a, const Chunk& ch, int nt, const WsSrc& src, int wave,
                                        int wm, int wn, int lane, int wr) {
  using S = Ws<V>;
  const int64_t N = a.N;
  const int nk = (int)(a.K / RBK);
  int ra[4], rb[4];
  const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = (2 * s + h) ^ swz8(l32);
    ra[s] = (wm * 32 + l32) * 8 + c;
    rb[s] = (wn * 64 + l32) * 8 + c;
  }
  f32x16 acc[WRB][WNB];
#pragma unroll
  for (int i = 0; i < WRB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  ws_kloop<V, MODE, NAL, NRB, R>(acc, src, nk, wr, ra, rb);

  // ---- epilogue: as the 256-row register-staged kernel, through a 16 KB
  // wave-private LDS region (free once every wave is past the K loop): 320 x
  // 256, two per 32 KB weight stage and waves 6-7 in the token row buffer;
  // 160 x 512, four per 64 KB weight stage
  rs_barrier();
  if constexpr (NRB > 0) {
    constexpr int NJ = MODE == MODE_GATEUP ? 1 : WNB;  // 32-column output blocks of this wave
    constexpr int LDSR = NJ * 32 + 8;                   // padded LDS row (elements)
    constexpr int CPRW = NJ * 4;                        // 16-byte chunks per output row
    static_assert(32 * LDSR * 2 <= 16 * 1024, "epilogue region");
    uint16_t* tile;
    if constexpr (V == 0) {
      static_assert(2 * 16 * 1024 <= S::BN * 128 && 2 * 16 * 1024 <= S::AL * 64 * 128, "epilogue region");
      u32x4* reg = wave < 2 ? sWB0 : wave < 4 ? sWB1 : wave < 6 ? sWB2 : sWA;
      tile = reinterpret_cast<uint16_t*>(reg) + (wave & 1) * (16 * 1024 / 2);
    } else {
      static_assert(4 * 16 * 1024 <= S::BN * 128, "epilogue region");
      u32x4* reg = wave < 4 ? sVB0 : sVB1;
      tile = reinterpret_cast<uint16_t*>(reg) + (wave & 3) * (16 * 1024 / 2);
    }
    uint16_t* out = static_cast<uint16_t*>(a.out);
    const int64_t n0 = MODE == MODE_GATEUP ? (int64_t)nt * (S::BN / 2) + wn * 32 : (int64_t)nt * S::BN + wn * 64;
    const bool odd = l32 & 1;
#pragma unroll
    for (int i = 0; i < NRB; ++i) {
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int p = 0; p < 4; p += 2) {
            float va, vb;
            if (MODE == MODE_GATEUP) {
              va = silu_f(acc[i][0][4 * g + p]) * acc[i][1][4 * g + p];
              vb = silu_f(acc[i][0][4 * g + p + 1]) * acc[i][1][4 * g + p + 1];
            } else {
              va = acc[i][jj][4 * g + p];
              vb = acc[i][jj][4 * g + p + 1];
            }
            // even lane: (row r, cols c, c+1); odd lane: (row r+1, cols c-1, c)
            const float x = lane_swap1(odd ? va : vb);
            const int r = 8 * g + 4 * h + p;
            const uint32_t w = odd ? pack_bf16x2(x, vb) : pack_bf16x2(va, x);
            const int lr = odd ? r + 1 : r;
            *reinterpret_cast<uint32_t*>(tile + lr * LDSR + jj * 32 + (l32 & ~1)) = w;
          }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
      const int rowb = (S::WM * i + wm) * 32;
#pragma unroll
      for (int q = 0; q < 32 * CPRW / kWave; ++q) {
        const int idx = q * kWave + lane;
        const int lr = idx / CPRW, c16 = idx % CPRW;
        const int row = rowb + lr;
        const int64_t n = n0 + c16 * 8;
        if (row < ch.nrows && n < N)
          store_out(out + ((int64_t)ch.row0 + row) * N + n, tile + lr * LDSR + c16 * 8, a.nt_out);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next block overwrites the region
    }
  }
}

template <int V, int MODE, int NA, int R>
__device__ __forceinline__ void ws_run(const GemmArgs& a, const Chunk& ch, int nt) {
  using S = Ws<V>;
  constexpr int NAL = (NA + 1) / 2;  // 64-row A groups fetched
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WN, wn = wave % S::WN;
  const bool shared = ch.group == a.E;
  const int64_t K = a.K, N = a.N;

  // loader: lane -> row (tid / 8) of each 64-row group, 16-byte chunk tid % 8
  // (A: the logical chunk, stored at its swizzled slot wr; B: the physical
  // slot, loaded from the logical chunk that belongs there)
  const int lrow = tid >> 3, lchunk = tid & 7;
  const int wr = lrow * 8 + (lchunk ^ swz8(lrow));
  WsSrc src;
  src.wave = wave;
  src.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.A), (short)0, -1, kBufFlags);
#pragma unroll
  for (int i = 0; i < S::AL; ++i) {
    const int rc = min(i * 64 + lrow, ch.nrows - 1);
    const int64_t row = (int64_t)ch.row0 + rc;
    int64_t sr = row;
    if (a.gather != nullptr) sr = shared ? row - a.shared_row0 : (int64_t)a.gather[row];
    src.aoff[i] = (uint32_t)((sr * K + lchunk * 8) * 2);  // A spans < 4 GiB (checked by the host)
  }
  const int64_t goff = shared ? 0 : (int64_t)ch.group * N * K;
  const int bchunk = lchunk ^ swz8(lrow);
  const uint16_t* W;
  if (MODE == MODE_GATEUP) {
    // B group j (tile rows 64 j .. 64 j + 63) is wave column j's 32 gate rows then
    // its 32 up rows; a loader wave's 8 rows are all gate (waves 0-3) or all up
    const bool up = wave >= 4;
    W = static_cast<const uint16_t*>(up ? (shared ? a.ws1 : a.w1) : (shared ? a.ws0 : a.w0)) + goff;
#pragma unroll
    for (int j = 0; j < S::BL; ++j)
      src.bgrp[j] = (uint32_t)(min((int64_t)nt * (S::BN / 2) + j * 32, N - 32) * K * 2);
    src.boff = (uint32_t)(((lrow & 31) * K + bchunk * 8) * 2);
  } else {
    W = static_cast<const uint16_t*>(shared ? a.ws0 : a.w0) + goff;
    // a group past N is clamped to the last 64 rows (loaded, never stored); N is a multiple of 64
#pragma unroll
    for (int j = 0; j < S::BL; ++j) src.bgrp[j] = (uint32_t)(min((int64_t)nt * S::BN + j * 64, N - 64) * K * 2);
    src.boff = (uint32_t)((lrow * K + bchunk * 8) * 2);
  }
  src.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(W), (short)0, -1, kBufFlags);

  if constexpr (S::WM == 1) {
    ws_wave<V, MODE, NAL, NA, R>(a, ch, nt, src, wave, wm, wn, lane, wr);
  } else {
    if (wm == 0) ws_wave<V, MODE, NAL, (NA + 1) / 2, R>(a, ch, nt, src, wave, wm, wn, lane, wr);
    else ws_wave<V, MODE, NAL, NA / 2, R>(a, ch, nt, src, wave, wm, wn, lane, wr);
  }
}

// Tile p of a launch over one chunk list, or (TWO) over both: list A's tiles,
// then list B's.  The down pass runs both lists on this kernel; as one launch
// it ends on one partly filled round of tiles instead of one per list.
template <int MODE, int V, int R, bool TWO = false>
__device__ __forceinline__ void ws_tile(const GemmArgs& a, int n_tiles, int p) {
  const int nva = *a.n_chunks * n_tiles;
  const int nv = TWO ? nva + *a.n_chunks_b * n_tiles : nva;
  int L;
  if (!xcd_map_cyclic(p, nv, SUPER * n_tiles, L)) return;
  const Chunk* list = a.chunks;
  if (TWO && L >= nva) {
    list = a.chunks_b;
    L -= nva;
  }
  int ci, nt;
  tile_of(L, n_tiles, list, ci, nt);
  const Chunk ch = list[ci];
  if constexpr (V == 0) {
    switch ((ch.nrows + 31) / 32) {
      case 1: ws_run<V, MODE, 1, R>(a, ch, nt); break;
      case 2: ws_run<V, MODE, 2, R>(a, ch, nt); break;
      case 3: ws_run<V, MODE, 3, R>(a, ch, nt); break;
      case 4: ws_run<V, MODE, 4, R>(a, ch, nt); break;
      case 5: ws_run<V, MODE, 5, R>(a, ch, nt); break;
      case 6: ws_run<V, MODE, 6, R>(a, ch, nt); break;
      case 7: ws_run<V, MODE, 7, R>(a, ch, nt); break;
      case 8: ws_run<V, MODE, 8, R>(a, ch, nt); break;
      case 9: ws_run<V, MODE, 9, R>(a, ch, nt); break;
      default: ws_run<V, MODE, 10, R>(a, ch, nt); break;
    }
    static_assert(Ws<0>::BM / 32 == 10, "row-block dispatch");
  } else {
    switch ((ch.nrows + 31) / 32) {
      case 1: ws_run<V, MODE, 1, R>(a, ch, nt); break;
      case 2: ws_run<V, MODE, 2, R>(a, ch, nt); break;
      case 3: ws_run<V, MODE, 3, R>(a, ch, nt); break;
      case 4: ws_run<V, MODE, 4, R>(a, ch, nt); break;
      default: ws_run<V, MODE, 5, R>(a, ch, nt); break;
    }
    static_assert(Ws<1>::BM / 32 == 5, "row-block dispatch");
  }
}

// The 320 x 256 tile (R = (nk - 2) % 3) and the 160 x 512 tile (R = (nk - 1) % 2).
template <int MODE, int R>
__global__ __launch_bounds__(WNT) void grouped_gemm_ws(GemmArgs a, int n_tiles) {
  ws_tile<MODE, 0, R>(a, n_tiles, blockIdx.x);
}
template <int R>
__global__ __launch_bounds__(WNT) void grouped_gemm_ws2(GemmArgs a, int n_tiles) {
  ws_tile<MODE_DOWN, 0, R, true>(a, n_tiles, blockIdx.x);
}
#ifndef MOE_WN_PERSIST
#define MOE_WN_PERSIST 1
#endif
// The 160 x 512 tile's K loops are short (capacity-limited layers have narrow
// H), so a tile's start-up weighs more than in the long-K tiles: one workgroup
// per CU walks the tiles p = blockIdx.x, + gridDim.x, ... (gridDim.x a
// multiple of the XCD count, so each workgroup keeps to its XCD's tiles), which
// saves the workgroup launches (about 1% of the Switch-style gate/up pass).
template <int MODE, int R>
__global__ __launch_bounds__(WNT) void grouped_gemm_wn(GemmArgs a, int n_tiles) {
  if constexpr (MOE_WN_PERSIST) {
    const int nv = *a.n_chunks * n_tiles;
    for (int p = blockIdx.x; p < nv; p += gridDim.x) {
      ws_tile<MODE, 1, R>(a, n_tiles, p);
      __syncthreads();  // the epilogue's LDS reads are done before the next tile's loads land
    }
  } else {
    ws_tile<MODE, 1, R>(a, n_tiles, blockIdx.x);
  }
}

// ------------------------------------------------------ bf16 streaming path
// Small batches (decode): every expert group has at most 16 rows, so the work is
// streaming each touched expert's weights once.  One wave owns 16 output columns
// (16 weight rows; gate/up: 16 gate + the same 16 up rows) of one chunk and runs
// v_mfma_f32_16x16x32_bf16 with the token rows padded to 16.  No barriers: the
// waves never share data.
//
// Weight loads: a large buffer read with the non-temporal hint streams at about
// 7.1 TB/s on this device against 6.2-6.3 TB/s without it, but only when every
// load instruction covers whole 128-byte lines; the MFMA operand layout (a lane
// holds 16 bytes of one of 16 rows, four lanes per row per instruction) covers
// half lines, and half-line non-temporal reads fall to about 5 TB/s.  So each
// lane loads one 16-byte piece of a whole line (eight lanes per row, eight rows
// per instruction, two instructions per 16 rows of a 64-wide K block), SP
// blocks in flight in registers; a block is then written to the wave's own LDS
// rows and read back in the operand layout.  The 16-byte slots of each 128-byte
// LDS row are XOR-swizzled by row / 2, so both the stores and the operand reads
// of any 16 lanes fall on 64 distinct banks.  The token rows (A) are tiny and
// cached: plain loads, straight into the operand layout.
#ifndef MOE_STREAM_SP
#define MOE_STREAM_SP 4
#endif
// Down pass: wave gw takes its K blocks from block gw * ROT (mod K / 64) on.
// Its weight rows are I = 2048 elements, 4 KB apart, and the waves, all in
// step, would otherwise read the same offset of every 4 KB row at once;
// starting each wave one block further spreads them.  The gate/up rows (H =
// 7168, 14 KB) stream faster in step, so that pass is left as it is.
#ifndef MOE_STREAM_ROT
#define MOE_STREAM_ROT 1
#endif
#ifndef MOE_STREAM_NT
#define MOE_STREAM_NT 1
#endif
constexpr int SW = 4;                 // waves per workgroup
constexpr int SKB = 64;               // K per block: one 128-byte line of a weight row
constexpr int SP = MOE_STREAM_SP;     // K blocks in flight per wave

// One 16-byte piece of a weight line, read once.
__device__ __forceinline__ uint4 ldw(const uint16_t* p) {
  if (MOE_STREAM_NT) {
    const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  return *reinterpret_cast<const uint4*>(p);
}
// LDS slot of 16-byte piece c of staged row r (16 rows x 8 slots per matrix).
__device__ __forceinline__ int stream_slot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <int MODE>
__global__ __launch_bounds__(SW * 64) void grouped_stream_bf16(GemmArgs a, int n_wt) {
  constexpr int M = MODE == MODE_GATEUP ? 2 : 1;  // weight matrices per block
  __shared__ uint4 stage[SW][M][16 * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int V = *a.n_chunks * n_wt;
  const int gw = blockIdx.x * SW + wave;
  if (gw >= V) return;  // whole wave; no barriers below
  const int ci = gw / n_wt, nt = gw % n_wt;
  const Chunk ch = a.chunks[ci];
  const bool shared = ch.group == a.E;
  const int64_t K = a.K, N = a.N;
  const int r16 = lane & 15, g4 = lane >> 4;

  // A: token row r16 of the chunk (clamped); substep s takes k = 32 s + 8 g4 .. + 8 of each block
  const int rc = min(r16, ch.nrows - 1);
  const int64_t row = (int64_t)ch.row0 + rc;
  int64_t src = row;
  if (a.gather != nullptr) src = shared ? row - a.shared_row0 : (int64_t)a.gather[row];
  const uint16_t* pa = static_cast<const uint16_t*>(a.A) + src * K + 8 * g4;
  // B: load i (0, 1) of a block takes row 16 nt + 8 i + (lane >> 3), piece lane & 7 (N is a multiple of 64)
  const int brow = lane >> 3, bpc = lane & 7;
  const int64_t goff = shared ? 0 : (int64_t)ch.group * N * K;
  const int64_t n = (int64_t)nt * 16 + brow;
  const uint16_t* pb[M];
  pb[0] = static_cast<const uint16_t*>(shared ? a.ws0 : a.w0) + goff + n * K + 8 * bpc;
  if constexpr (M == 2) pb[1] = static_cast<const uint16_t*>(shared ? a.ws1 : a.w1) + goff + n * K + 8 * bpc;

  f32x4 acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nkb = (int)(K / SKB);  // K is a multiple of 64
  const int rot = (MODE == MODE_DOWN && nkb > 0) ? (int)(((int64_t)gw * MOE_STREAM_ROT) % nkb) : 0;
  auto koff = [&](int b) {  // K offset of the wave's b-th block: the blocks taken from block rot on, wrapping
    int r = b + rot;
    r -= r >= nkb ? nkb : 0;
    return (int64_t)r * SKB;
  };
  uint4 ra[SP][2], rb[SP][M][2];
  auto load = [&](int p, int b) {
    const int64_t ko = koff(b);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) ra[p][s2] = *reinterpret_cast<const uint4*>(pa + ko + 32 * s2);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < 2; ++i) rb[p][m][i] = ldw(pb[m] + 8 * i * K + ko);
  };
  // store slots of this lane's two pieces, read slots of its two operand pieces
  const int wslot0 = stream_slot(brow, bpc), wslot1 = stream_slot(8 + brow, bpc);
  const int rslot0 = stream_slot(r16, g4), rslot1 = stream_slot(r16, 4 + g4);
  // One block: stage its weight lines, read them back as operands, multiply.
  // Blocks past the end (K / 64 not a multiple of SP) multiply a zero A operand.
  auto block = [&](int p, int kb) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      stage[wave][m][wslot0] = rb[p][m][0];
      stage[wave][m][wslot1] = rb[p][m][1];
    }
    const bool live = kb < nkb;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint4 a4 = live ? ra[p][s2] : make_uint4(0u, 0u, 0u, 0u);
      const bf16x8 av = __builtin_bit_cast(bf16x8, a4);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4 bv = stage[wave][m][s2 ? rslot1 : rslot0];
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bv), acc[m], 0, 0, 0);
      }
    }
  };
  if (nkb > 0) {
    // SP blocks in flight: the steady loop refills each register set as soon
    // as its block is used, unconditionally (so the compiler's wait counts are
    // exact); the last SP blocks issue no loads.
    const int last = (nkb - 1) / SP * SP;  // first block of the last round
#pragma unroll
    for (int p = 0; p < SP; ++p) load(p, min(p, nkb - 1));
    for (int kb0 = 0; kb0 < last; kb0 += SP) {
#pragma unroll
      for (int p = 0; p < SP; ++p) {
        block(p, kb0 + p);
        load(p, min(kb0 + p + SP, nkb - 1));
      }
    }
#pragma unroll
    for (int p = 0; p < SP; ++p) block(p, last + p);
  }
  // lane holds output column 16 nt + r16 for token rows 4 g4 + q
  const int64_t ncol = (int64_t)nt * 16 + r16;
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rr = 4 * g4 + q;
    if (rr >= ch.nrows) continue;
    const int64_t orow = (int64_t)ch.row0 + rr;
    if (MODE == MODE_GATEUP)
      out[orow * N + ncol] = f32_to_bf16(silu_f(acc[0][q]) * acc[M - 1][q]);
    else
      out[orow * N + ncol] = f32_to_bf16(acc[0][q]);
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
  if (dtype == MOE_BF16 && a.bm == kGemvBM) {
    const int n_wt = (int)(a.N / 16);
    const int64_t grid = (a.max_chunks * n_wt + SW - 1) / SW;
    hipLaunchKernelGGL(grouped_stream_bf16<MODE>, dim3((unsigned)grid), dim3(SW * 64), 0, s, a, n_wt);
  } else if (dtype == MOE_BF16 && MODE == MODE_GATEUP && a.bm == kWideRows && rs_fits(a)) {
    if constexpr (MODE == MODE_GATEUP) {  // (the down pass takes the 320-row kernel)
      constexpr int BN = Ws<1>::BN;
      const int n_tiles = (int)((a.N + BN / 2 - 1) / (BN / 2));
      int64_t grid = ((a.max_chunks * n_tiles + kXcds - 1) / kXcds) * kXcds;
      if (MOE_WN_PERSIST) grid = std::min<int64_t>(grid, kNumCUs);
      static_assert(kNumCUs % kXcds == 0, "persistent grid");
      if ((a.K / RBK - 1) % 2)
        hipLaunchKernelGGL((grouped_gemm_wn<MODE, 1>), dim3((unsigned)grid), dim3(WNT), 0, s, a, n_tiles);
      else
        hipLaunchKernelGGL((grouped_gemm_wn<MODE, 0>), dim3((unsigned)grid), dim3(WNT), 0, s, a, n_tiles);
    }
  } else if (dtype == MOE_BF16 && a.bm == RBM && rs_fits(a)) {
    const int n_tiles = (int)(MODE == MODE_GATEUP ? (a.N + 127) / 128 : (a.N + RBN - 1) / RBN);
    const int64_t grid = ((a.max_chunks * n_tiles + kXcds - 1) / kXcds) * kXcds;
    if ((a.K / RBK) % 2)
      hipLaunchKernelGGL((grouped_gemm_rs<MODE, true>), dim3((unsigned)grid), dim3(RNT), 0, s, a, n_tiles);
    else
      hipLaunchKernelGGL((grouped_gemm_rs<MODE, false>), dim3((unsigned)grid), dim3(RNT), 0, s, a, n_tiles);
  } else if (dtype == MOE_BF16 && MOE_GEMM_WS && a.bm == WBM && rs_fits(a)) {
    constexpr int BN = Ws<0>::BN;
    const int n_tiles = (int)(MODE == MODE_GATEUP ? (a.N + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN);
    const int64_t grid = ((a.max_chunks * n_tiles + kXcds - 1) / kXcds) * kXcds;
    switch ((a.K / RBK - 2) % 3) {
      case 0: hipLaunchKernelGGL((grouped_gemm_ws<MODE, 0>), dim3((unsigned)grid), dim3(WNT), 0, s, a, n_tiles); break;
      case 1: hipLaunchKernelGGL((grouped_gemm_ws<MODE, 1>), dim3((unsigned)grid), dim3(WNT), 0, s, a, n_tiles); break;
      default: hipLaunchKernelGGL((grouped_gemm_ws<MODE, 2>), dim3((unsigned)grid), dim3(WNT), 0, s, a, n_tiles); break;
    }
  } else if (dtype == MOE_BF16) {
    const int n_tiles = (int)(MODE == MODE_GATEUP ? (a.N + 127) / 128 : (a.N + BN - 1) / BN);
    const int64_t grid = ((a.max_chunks * n_tiles + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL(grouped_gemm_bf16<MODE>, dim3((unsigned)grid), dim3(NT), 0, s, a, n_tiles);
  } else {
    const int n_tiles = (int)(MODE == MODE_GATEUP ? a.N / 32 : (a.N + 63) / 64);
    const int64_t grid = ((a.max_chunks * n_tiles + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL(grouped_gemm_f32<MODE>, dim3((unsigned)grid), dim3(256), 0, s, a, n_tiles);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup(const GemmArgs& a, int dtype, hipStream_t s) { return launch_gemm<MODE_GATEUP>(a, dtype, s); }
// The down pass (K = I) runs the 256-row list's chunks on the 320-row kernel
// as well (they have at most 256 rows): measured 1-2% faster there on the
// DeepSeek-V3 and Mixtral shapes, where the gate/up pass (K = H) is 8% faster
// with the 256-row kernel taking them.  The 160-row list's chunks go there
// too: a 160 x 512 down tile would leave half the CUs of a capacity-limited
// layer idle (H / 512 n-tiles per expert).
#ifndef MOE_DOWN_ON_WS
#define MOE_DOWN_ON_WS 1
#endif
hipError_t launch_down(const GemmArgs& a, int dtype, hipStream_t s) {
  if (MOE_DOWN_ON_WS && MOE_GEMM_WS && dtype == MOE_BF16 && (a.bm == kGemmBMrs || a.bm == kGemmBMwn) && rs_fits(a)) {
    GemmArgs b = a;
    b.bm = kGemmBMdl;
    return launch_gemm<MODE_DOWN>(b, dtype, s);
  }
  return launch_gemm<MODE_DOWN>(a, dtype, s);
}

#ifndef MOE_DOWN_ONE_LAUNCH
#define MOE_DOWN_ONE_LAUNCH 1
#endif
// One launch pays where a pass spans many rounds of tiles over the CUs: two
// launches end on two partly filled rounds (the DeepSeek-V3-shaped down pass:
// 13.6 + 17.3 rounds, 2.27 -> 2.23 ms as one launch).  A pass of a round or two
// per list keeps each launch's tiles in step, so that the n-tiles of a chunk
// share its token rows in L2; merged, the second round starts staggered (the
// Mixtral-shaped down pass, one round per list: 0.825 -> 0.85 ms).  The host
// bound on the tile count decides.
constexpr int64_t kOneLaunchMinRounds = 8;
bool launch_down_both(const GemmArgs& a, int dtype, hipStream_t s, hipError_t& err) {
  if (!(MOE_DOWN_ONE_LAUNCH && MOE_DOWN_ON_WS && MOE_GEMM_WS && dtype == MOE_BF16 && a.chunks_b != nullptr &&
        rs_fits(a)))
    return false;
  constexpr int BN = Ws<0>::BN;
  const int n_tiles = (int)((a.N + BN - 1) / BN);
  if (a.max_chunks * n_tiles < kOneLaunchMinRounds * kNumCUs) return false;
  const int64_t grid = ((a.max_chunks * n_tiles + kXcds - 1) / kXcds) * kXcds;
  switch ((a.K / RBK - 2) % 3) {
    case 0: hipLaunchKernelGGL((grouped_gemm_ws2<0>), dim3((unsigned)grid), dim3(WNT), 0, s, a, n_tiles); break;
    case 1: hipLaunchKernelGGL((grouped_gemm_ws2<1>), dim3((unsigned)grid), dim3(WNT), 0, s, a, n_tiles); break;
    default: hipLaunchKernelGGL((grouped_gemm_ws2<2>), dim3((unsigned)grid), dim3(WNT), 0, s, a, n_tiles); break;
  }
  err = hipGetLastError();
  return true;
}

}  // namespace moe
