// Internal declarations shared by the HIP translation units of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <functional>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumCUs = 256;      // MI355X compute units (32 per XCD)
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kMaxK = 16;
constexpr int kMaxE = 1024;

// Row-chunk of one expert group handled by one grouped-GEMM M-tile.
struct Chunk {
  int32_t group;   // expert id; == E for the shared expert
  int32_t row0;    // first row in the permuted row space
  int32_t nrows;   // rows in this chunk (1..BM)
  int32_t gfirst;  // index of the first chunk of this group in the list
  int32_t gcount;  // chunks of this group
  int32_t pad[3];
};

// M-tile heights of the bf16 grouped GEMM chunk lists: 256 rows (register-
// staged, one wave per SIMD) and 320 rows (register-staged with two waves per
// SIMD where its 32-bit offsets fit, else direct-to-LDS).
#ifndef MOE_GEMM_RS
#define MOE_GEMM_RS 1
#endif
#ifndef MOE_GEMM_WS
#define MOE_GEMM_WS 1
#endif
constexpr int kGemmBMrs = 256;
constexpr int kGemmBMdl = 320;
// Chunk height of layers whose routed groups hold at most this many rows (an
// expert capacity) and that have no shared expert: one list of 160-row chunks,
// whose gate/up pass runs a 160 x 512 tile.
#ifndef MOE_GEMM_WN
#define MOE_GEMM_WN 1
#endif
constexpr int kGemmBMwn = 160;
// M-tile height of the fp32 grouped GEMM.
constexpr int kGemmBMf32 = 64;
// Row chunks of the bf16 weight-streaming path used for small batches (decode).
constexpr int kGemvBM = 16;
constexpr int64_t kGemvMaxT = 16;

// Chunks of one group that the GEMM tile order interleaves per n-tile (they
// share each weight tile, read once into one XCD's L2).
constexpr int kChunkSuper = 4;

// How the dispatch step cuts expert groups into row chunks: one list of bm_a-row
// chunks (bm_b == 0), or two lists, A of bm_a-row chunks at chunks[0] and B of
// bm_b-row chunks at chunks[off_b], each group going to the list where it costs
// less (decided on the device from its row count).  cus (the device's compute
// units) and nt (gate/up tiles per chunk) let the dispatch step place the
// shared group's gate/up chunks so that both lists end on nearly full rounds
// of tiles (0: unknown, the shared group's gate/up chunks all go to list A).
struct ChunkCut {
  int bm_a;
  int bm_b;
  int64_t off_b;
  int cus = 0;
  int nt = 0;
};

// Max chunk-list entries for `rows_max` routed rows over E groups (+ shared rows).
int64_t max_chunks(int64_t rows_max, int64_t E, int64_t shared_rows, int bm);

// Chunk lists of a layer with at most `routed` routed rows over E groups plus
// `shared` shared rows: the streaming path when every group fits one 16-row
// chunk (T <= 16), 64-row chunks for fp32; for bf16 two lists (256-row and
// 320-row tiles) when the register-staged kernels' limits hold (both
// contractions at least 128 long, 32-bit buffer offsets covering x [T, H], the
// row space [rows, H] and h [rows, I]), else the 320-row tile alone.
// max_a / max_b: capacities of the two lists.  group_max (-1: unknown) bounds
// the rows of one routed group: at most 256 rows, every group takes the
// 256-row list (and so does the shared group, which never makes the other list
// on its own), so the 320-row list is left out and its launches skipped; at
// most 160 rows with no shared rows, the one list is cut to 160-row chunks.
struct ChunkPlan {
  ChunkCut cut;
  int64_t max_a, max_b;
};
inline ChunkPlan chunk_plan(const moe_config& c, int64_t routed, int64_t shared, int64_t group_max = -1) {
  ChunkPlan p{};
  const int64_t rows = routed + shared, lim = int64_t(1) << 32;
  int bm_a = kGemmBMdl, bm_b = 0;
  if (c.dtype != MOE_BF16) {
    bm_a = kGemmBMf32;
  } else if (c.T <= kGemvMaxT) {
    bm_a = kGemvBM;
  } else if (MOE_GEMM_RS && c.H >= 128 && c.I >= 128 && std::max<int64_t>(c.T, rows) * c.H * 2 < lim &&
             rows * c.I * 2 < lim && c.H * c.I * 2 < lim) {
    bm_a = kGemmBMrs;
    bm_b = (group_max >= 0 && group_max <= kGemmBMrs) ? 0 : kGemmBMdl;
    if (MOE_GEMM_WN && group_max >= 0 && group_max <= kGemmBMwn && shared == 0) bm_a = kGemmBMwn;
  }
  p.max_a = max_chunks(routed, c.E, shared, bm_a);
  p.max_b = bm_b ? max_chunks(routed, c.E, shared, bm_b) : 0;
  p.cut = ChunkCut{bm_a, bm_b, p.max_a};
  return p;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);  // gfx950: v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// ---- launches (each returns hipGetLastError() of its launch) ----

// Selection options of the router kernels and their optional dense output.
struct RouteSel {
  const float* sbias;  // [E] selection-only expert bias, or NULL
  int n_group;         // expert groups of the group limit (0: none)
  int topk_group;      // groups kept per token
  float* scores;       // [T, E] gate score of every expert, or NULL
};
inline RouteSel route_sel_of(const moe_config& c, const float* sbias, float* scores) {
  return RouteSel{sbias, c.n_group, c.topk_group, scores};
}

// Router GEMM + gate + top-k.  x, w: bf16 or fp32 per dtype.
hipError_t launch_route(const moe_config& c, const void* x, const void* w, const float* bias, const RouteSel& rs,
                        int32_t* topk_idx, float* topk_w, hipStream_t s);

// Router partial logits (bf16): part[s][t][0 .. 32 ceil(E/32)) float32 over
// route_partial_slices(c) slices of H, in `part` (route_scratch_bytes).
int route_partial_slices(const moe_config& c);
size_t route_scratch_bytes(const moe_config& c);
hipError_t launch_route_partials(const moe_config& c, const void* x, const void* w, float* part, hipStream_t s);

// Split-K router (bf16): partial logits in `scratch` (route_scratch_bytes), then
// a per-token reduce + gate + top-k.  fp32 configs fall back to launch_route.
hipError_t launch_route_split(const moe_config& c, const void* x, const void* w, const float* bias,
                              const RouteSel& rs, int32_t* topk_idx, float* topk_w, void* scratch, hipStream_t s);

// Routing statistics: P_i (mean score), f_i (routed fraction) and E * sum f_i P_i
// from counts [E] and scores [T, E]; `part` holds stats_scratch_bytes(c).
size_t stats_scratch_bytes(const moe_config& c);
hipError_t launch_balance_stats(const moe_config& c, const int32_t* counts, const float* scores, float* mean,
                                float* frac, float* balance, void* part, hipStream_t s);
// score_bias[e] += gamma * sign(mean load - counts[e]).
hipError_t launch_bias_update(const moe_config& c, const int32_t* counts, float gamma, float* score_bias,
                              hipStream_t s);

// Dispatch scratch sizes (bytes) for T tokens, k slots and E experts.
size_t dispatch_scratch_bytes(int64_t T, int64_t k, int64_t E);

// The layer's routing and dispatch (bf16): router partials, the select step
// (sum of the partials, gate, top-k) with the dispatch's block step, then the
// expert scan and the row maps and chunk lists; `routed` runs after the select
// step (the stage boundary between routing and dispatch).  Batches of <= 16
// tokens do the select step and the whole dispatch in one launch
// (route_dispatch_fused).  rscratch: route_scratch_bytes; dscratch:
// dispatch_scratch_bytes.
bool route_dispatch_fused(const moe_config& c);
hipError_t launch_route_dispatch(const moe_config& c, const void* x, const void* w, const float* bias,
                                 const RouteSel& rs, int32_t* topk_idx, float* topk_w, void* rscratch, int64_t cap,
                                 int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* token_of_row,
                                 void* dscratch, Chunk* chunks, int32_t* n_chunks, const ChunkCut& cut,
                                 int64_t shared_rows, int64_t shared_row0, hipStream_t s,
                                 const std::function<hipError_t()>& routed);

// Histogram + scan + capacity + row maps; also writes the chunk lists of the
// routed groups (and the shared group when shared_rows > 0, starting at
// shared_row0 in the row space); n_chunks[0..1] receive the list sizes of the
// gate/up pass, n_chunks[2..3] those of the down pass (the shared group's chunks
// can sit in a different list in each).
hipError_t launch_dispatch(int64_t T, int64_t k, int64_t E, int64_t cap, const int32_t* topk_idx,
                           int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                           int32_t* token_of_row, void* scratch, Chunk* chunks, int32_t* n_chunks,
                           const ChunkCut& cut, int64_t shared_rows, int64_t shared_row0, hipStream_t s);

// Chunk lists from a device offsets array (stage API).
hipError_t launch_chunks_from_offsets(const int32_t* offsets, int64_t E, Chunk* chunks,
                                      int32_t* n_chunks, const ChunkCut& cut, hipStream_t s);

// x_perm[row] = x[token_of_row[row]] for row < offsets[E].
hipError_t launch_gather(const void* x, const int32_t* token_of_row, const int32_t* offsets,
                         int64_t E, int64_t rows_max, int64_t H, int dtype, void* x_perm,
                         hipStream_t s);

struct GemmArgs {
  const void* A;            // activations: x (gathered) or x_perm / h (direct rows)
  const int32_t* gather;    // token_of_row, or NULL: row r of A is row r of the row space
  int64_t shared_row0;      // first row of the shared group in the row space (gather mode)
  const Chunk* chunks;
  const int32_t* n_chunks;  // device count of valid chunks
  // A second chunk list run in the same launch after the first (the down pass
  // over both lists), or NULL; max_chunks then bounds both lists together.
  const Chunk* chunks_b = nullptr;
  const int32_t* n_chunks_b = nullptr;
  int64_t max_chunks;       // grid bound
  const void* w0;           // gate (gate/up pass) or down weights, [E, N, K]
  const void* w1;           // up weights (gate/up pass)
  const void* ws0;          // shared expert's gate or down
  const void* ws1;          // shared expert's up
  int64_t E;
  int64_t K;                // contraction length (H or I)
  int64_t N;                // output columns (I or H)
  void* out;                // [rows, N]
  int bm;                   // chunk height the list was cut to (selects the kernel)
  int64_t a_rows = 0;       // rows of A addressable through `gather` / the row space
  // Output stores bypass the caches (written once, read once by the next pass):
  // set for h, and for y_perm when it is larger than the last-level cache
  // (smaller ones are read back from it by the combine).
  bool nt_out = false;
  // FP8 weights (w0/w1/ws0/ws1 then hold E4M3 codes): float32 scales per
  // kFp8Block x kFp8Block block, [E, N/128, K/128] and [N/128, K/128] (shared)
  const float* sc0 = nullptr;
  const float* sc1 = nullptr;
  const float* ssc0 = nullptr;
  const float* ssc1 = nullptr;
};

// Last-level (MALL) cache size of the MI355X: outputs larger than this are
// stored non-temporally.
constexpr int64_t kLastLevelCacheBytes = int64_t(256) << 20;
hipError_t launch_gateup(const GemmArgs& a, int dtype, hipStream_t s);
hipError_t launch_down(const GemmArgs& a, int dtype, hipStream_t s);
// The down pass over both chunk lists in one launch of the 320-row kernel
// (a.chunks / a.n_chunks, then a.chunks_b / a.n_chunks_b; a.max_chunks bounds
// both).  False, with nothing launched, where that kernel does not take the
// pass (then each list is launched on its own).
bool launch_down_both(const GemmArgs& a, int dtype, hipStream_t s, hipError_t& err);

// FP8 (E4M3) weights, bf16 activations, batches of <= kGemvMaxT tokens.
constexpr int kFp8Block = 128;
hipError_t launch_gateup_fp8(const GemmArgs& a, hipStream_t s);
hipError_t launch_down_fp8(const GemmArgs& a, hipStream_t s);
// Block-scaled E4M3 quantisation of G matrices [N, K] (bf16 or fp32 per dtype).
hipError_t launch_quantize_fp8(const void* w, int dtype, int64_t G, int64_t N, int64_t K, uint8_t* codes,
                               float* scales, hipStream_t s);

// y[t] = sum over slots j < k with row_of_slot[t*k+j] >= 0 of scale * topk_w[t*k+j]
// * y_perm[row] (+ y_shared[t]); k up to kMaxE.
hipError_t launch_combine(const void* y_perm, const int32_t* row_of_slot, const float* topk_w,
                          const void* y_shared, void* y, int64_t T, int64_t H, int64_t k,
                          int dtype, hipStream_t s, float scale = 1.f);

// Calibration: MFMA-only kernel (iters rounds of 4 chains per wave), its
// flop count and its sink length.
int64_t mfma_peak_flops(int64_t iters);
int64_t mfma_peak_sink_len();
hipError_t launch_mfma_peak(int iters, bool varied, float* sink, hipStream_t s);
// Calibration: one read of nblocks 32 KiB blocks of buf; sink holds
// hbm_read_sink_len() XORs of the words each workgroup read.
constexpr int64_t kReadBlockBytes = 32768;
int64_t hbm_read_sink_len();
hipError_t launch_hbm_read(const void* buf, int64_t nblocks, uint32_t* sink, hipStream_t s);

// Expert choice: chunk list of E groups of C rows each (+ shared rows), and the
// per-expert top-C selection from scores [T, E].
hipError_t launch_chunks_uniform(int64_t E, int64_t C, int64_t shared_rows, int64_t shared_row0, Chunk* chunks,
                                 int32_t* n_chunks, const ChunkCut& cut, hipStream_t s);
hipError_t launch_ec_select(const float* scores, int64_t T, int64_t E, int64_t C, int32_t* token_of_row,
                            int32_t* row_of_pair, hipStream_t s);

}  // namespace moe
