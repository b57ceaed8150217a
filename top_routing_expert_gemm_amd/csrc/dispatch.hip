// Histogram + stable scan + capacity, row maps, chunk lists and the row gather.
//
// Sources: niuwancheng.cn "10. 混合专家 MoE：总参数与激活参数", section
// "把一个大 FFN 换成一组小 FFN" (the rows of each expert are collected and run as
// one batched GEMM) and section "负载不均：路由坍缩与丢 token" (capacity =
// tokens / experts x factor, rounded up; overflow tokens skip the expert);
// amazingdata.cn "moe-routing-hardest" (expert-capacity paragraph).
//
// Determinism: the rank of an assignment inside its expert is the number of
// earlier (token, slot) assignments to that expert.  It is computed without
// relying on the order of atomics:
//   1. blocks      the assignments are cut into blocks of consecutive
//                  (token, slot) pairs; one wave per block walks them in order,
//                  64 at a time; lanes with equal experts are grouped by a ballot
//                  match and ranked by lane order; a per-block LDS counter per
//                  expert carries the count across steps.  Emits the local rank
//                  and the block histogram.  In the layer this runs inside the
//                  router's select kernel (a block = the 16 tokens of one
//                  workgroup); the stage entry point has its own kernel.
//   2. expert scan one workgroup per expert: exclusive scan of its block counts
//                  (block bases) and its demand count.
//   3. finalize    every block's workgroup scans the E loads (min(count, cap))
//                  into offsets itself; rank = block base + local rank; kept iff
//                  rank < cap; row_of_slot / token_of_row.  The first workgroup
//                  also writes offsets and the GEMM chunk lists (the shared
//                  group's chunks placed per pass, with four list counts).
// Batches of at most 1024 assignments do all of it in one workgroup (for the
// layer's decode batches, together with the router's select step).
#include <functional>

#include "common.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;

// Assignments per histogram block: 256 (four 64-wide steps of one wave), doubled
// until there are at most 4096 blocks.
inline int64_t hist_chunk(int64_t Tk) {
  int64_t ch = 256;
  while ((Tk + ch - 1) / ch > 4096) ch *= 2;
  return ch;
}
inline int64_t hist_blocks(int64_t Tk) {
  const int64_t ch = hist_chunk(Tk);
  return Tk == 0 ? 1 : (Tk + ch - 1) / ch;
}
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// One wave ranks n assignments in order: id_at(i) is the expert of assignment
// i; rank_at(i, r) receives its rank r among the earlier assignments to the
// same expert, counted on from cnt[e] (LDS, one counter per expert, advanced
// past these assignments), or -1 for an id outside [0, E) (a violated
// precondition: skipped, never used as an index).
template <typename Id, typename Out>
__device__ void wave_rank(Id id_at, Out rank_at, int64_t n, int E, int32_t* cnt) {
  const int lane = threadIdx.x & (kWave - 1);
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = 0; base < n; base += 64) {
    const int64_t i = base + lane;
    int e = i < n ? id_at(i) : 0;
    const bool valid = i < n && e >= 0 && e < E;
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bal = __ballot(valid && on);
      peers &= on ? bal : ~bal;
    }
    const int before = __popcll(peers & lt);
    const int old = valid ? cnt[e] : 0;
    __builtin_amdgcn_wave_barrier();  // every lane has read its counter before the leaders update
    if (valid && before == 0) cnt[e] = old + __popcll(peers);
    if (i < n) rank_at(i, valid ? old + before : -1);
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(64) void hist_rank_kernel(const int32_t* __restrict__ idx, int64_t Tk,
                                                       int E, int64_t CH, int32_t* __restrict__ blk_counts,
                                                       int32_t* __restrict__ rank_tmp) {
  __shared__ int32_t cnt[kMaxE];
  const int64_t b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  const int64_t begin = b * CH, n = min(begin + CH, Tk) - begin;
  wave_rank([&](int64_t i) { return idx[begin + i]; }, [&](int64_t i, int r) { rank_tmp[begin + i] = r; }, n, E,
            cnt);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64) blk_counts[b * E + e] = cnt[e];
}

// Inclusive scan over the block (one value per thread, blockDim.x == kScanThreads):
// a shuffle scan within each wave, then each wave adds the totals of the waves
// before it (tmp[0 .. kScanThreads / 64) holds them); two barriers in all.
__device__ int block_inclusive_scan(int v, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  for (int w = 0; w < wave; ++w) x += tmp[w];
  __syncthreads();  // tmp is free again when this returns
  return x;
}

// Which list a group of L rows goes to.  With one list (bm_b == 0) every group
// is cut to bm_a rows.  With two (the 256-row tile in list A, the 320-row tile
// in list B), a list-A chunk costs about 0.88-0.91 of a list-B chunk (measured
// on the DeepSeek-V3, Mixtral and Switch shapes; 0.91 with the current 320-row
// kernel, expert choice with every group on one tile or the other), so a group
// takes list A unless that needs more chunks than the lower cost saves (a group
// of 257..320 rows: two chunks instead of one).
__device__ __forceinline__ bool takes_list_a(int64_t L, const ChunkCut& cut) {
  if (cut.bm_b == 0) return true;
  const int64_t na = (L + cut.bm_a - 1) / cut.bm_a, nb = (L + cut.bm_b - 1) / cut.bm_b;
  return 22 * na <= 25 * nb;
}

// Chunk lists of E groups with given loads and first rows, then (optionally) the
// shared group over rows shared_row0 .. shared_row0 + shared_rows - 1.  A group
// of `load` rows takes n = ceil(load / bm) chunks of its list's height bm, of
// balanced size (chunk c holds rows [c load / n, (c + 1) load / n)), so the
// workgroups that stream the same weight tile for one group do equal work and
// stay in step.  List A starts at chunks[0], list B at chunks[cut.off_b]; each
// list is compact and expert-ordered (shared group last), n_chunks[0] and
// n_chunks[1] count them.  The shared group goes to list B only when routed
// groups already went there.
__device__ void emit_chunks(int e_valid, int load, int row0, int E, const ChunkCut& cut, int64_t shared_rows,
                            int64_t shared_row0, Chunk* chunks, int32_t* n_chunks, int* tmp) {
  const int tid = threadIdx.x;
  const bool in_a = takes_list_a(load, cut);
  const int bm = in_a ? cut.bm_a : cut.bm_b;
  const int nch = e_valid ? (load + bm - 1) / bm : 0;
  const int incl_a = block_inclusive_scan(in_a ? nch : 0, tmp);
  const int incl_b = block_inclusive_scan(in_a ? 0 : nch, tmp);
  const int base = in_a ? incl_a - nch : incl_b - nch;
  Chunk* list = in_a ? chunks : chunks + cut.off_b;
  for (int c = 0; c < nch; ++c) {
    const int r0 = (int)((int64_t)c * load / nch), r1 = (int)((int64_t)(c + 1) * load / nch);
    Chunk ck;
    ck.group = tid;
    ck.row0 = row0 + r0;
    ck.nrows = r1 - r0;
    ck.gfirst = base;
    ck.gcount = nch;
    ck.pad[0] = ck.pad[1] = ck.pad[2] = 0;
    list[base + c] = ck;
  }
  __shared__ int total_a, total_b;
  if (tid == kScanThreads - 1) {
    total_a = incl_a;
    total_b = incl_b;
  }
  __syncthreads();
  // The shared group.  Its chunks share one weight tile per n-tile, which the
  // tile order streams once per group of chunks, so the 320-row list's fewer
  // weight streams buy it little; the down pass (the 320-row kernel over both
  // lists) takes it as fewer, taller chunks of list B, the gate/up pass mostly
  // as chunks of list A (the 256-row kernel has the higher rate per row).  Each
  // gate/up launch ends on a partly filled round of tiles, so the gate/up pass
  // takes the first j of list B's shared chunks as well, and list A covers
  // the rows after them: j is the count (0 .. all, in whole groups of
  // kChunkSuper chunks, so that the remaining shared chunks start on a group
  // boundary and the tile order keeps each of their weight tiles within one
  // XCD) that minimises the rounds of tiles of both launches (cus compute
  // units, nt tiles per chunk), each round weighted by its kernel's cost per
  // chunk (22 : 25, as above).
  // Layout: list A = [routed A][shared rows rb .. R in nsa chunks], list B =
  // [routed B][shared rows 0 .. R in nsb chunks, the first j one weight-sharing
  // group, the rest another].  Counts: n_chunks[0..1] (gate/up) total_a + nsa,
  // total_b + j; n_chunks[2..3] (down) total_a, total_b + nsb.  With one list,
  // or no routed group in list B (a launch of only the shared chunks would
  // leave most CUs idle), list A holds the shared chunks for both passes.
  const bool split = cut.bm_b != 0 && total_b > 0;
  const int64_t R = shared_rows;
  const int nsb = split ? (int)((R + cut.bm_b - 1) / cut.bm_b) : 0;
  // One wave evaluates the candidates on wave-uniform (scalar) values and
  // hands j to the others through LDS.
  __shared__ int sh_j;
  if (tid < kWave) {
    int j = 0;
    const int ta = __builtin_amdgcn_readfirstlane(total_a), tb = __builtin_amdgcn_readfirstlane(total_b);
    if (split && R > 0 && cut.cus > 0 && cut.nt > 0) {
      // The rounds of list A fall as j grows, those of list B rise, so for
      // each round count of list B the largest admissible j is the only
      // candidate: at most a few, each a few exact integer divisions (no
      // loop over every j on this critical path).  Ties keep the smaller j.
      const int r32 = (int)R, nt = cut.nt, cus = cut.cus, bma = cut.bm_a;
      auto cost = [&](int jj) {
        const int ra = r32 - (int)((int64_t)jj * r32 / nsb);
        const int na = ta + (ra + bma - 1) / bma;
        return 22 * ((na * nt + cus - 1) / cus) + 25 * (((tb + jj) * nt + cus - 1) / cus);
      };
      int best = cost(0);
      const int k0 = (tb * nt + cus - 1) / cus, k1 = ((tb + nsb) * nt + cus - 1) / cus;
      for (int kk = k0; kk <= k1; ++kk) {
        int jm = min(nsb, kk * cus / nt - tb);
        if (jm < nsb) jm = jm / kChunkSuper * kChunkSuper;  // whole groups of kChunkSuper (or all)
        if (jm <= 0) continue;
        const int cj = cost(jm);
        if (cj < best) {
          best = cj;
          j = jm;
        }
      }
    }
    if (tid == 0) sh_j = j;
  }
  __syncthreads();
  const int j = sh_j;
  const int64_t rb = nsb > 0 ? j * R / nsb : 0;  // shared rows the gate/up pass takes from list B
  const int nsa = (int)((R - rb + cut.bm_a - 1) / cut.bm_a);
  // chunk c of n over shared rows [lo, hi), in a weight-sharing group of gc chunks from gf
  auto put = [&](Chunk* list, int base, int n, int64_t lo, int64_t hi, int gf0, int gc0, int gf1, int gc1, int cut_at) {
    for (int c = tid; c < n; c += kScanThreads) {
      const int64_t r0 = lo + c * (hi - lo) / n, r1 = lo + (c + 1) * (hi - lo) / n;
      Chunk ck;
      ck.group = E;
      ck.row0 = (int)(shared_row0 + r0);
      ck.nrows = (int)(r1 - r0);
      ck.gfirst = c < cut_at ? gf0 : gf1;
      ck.gcount = c < cut_at ? gc0 : gc1;
      ck.pad[0] = ck.pad[1] = ck.pad[2] = 0;
      list[base + c] = ck;
    }
  };
  put(chunks, total_a, nsa, rb, R, total_a, nsa, total_a, nsa, nsa);
  if (split) put(chunks + cut.off_b, total_b, nsb, 0, R, total_b, j, total_b + j, nsb - j, j);
  if (tid == 0) {
    n_chunks[0] = total_a + nsa;
    n_chunks[1] = split ? total_b + j : (cut.bm_b != 0 ? total_b : 0);
    n_chunks[2] = split ? total_a : total_a + nsa;
    n_chunks[3] = split ? total_b + nsb : n_chunks[1];
  }
}

// Per expert (one workgroup each): exclusive scan of its nb block counts in
// block order, written back as the block bases, and its demand count.
constexpr int kEsThreads = 256;
__global__ __launch_bounds__(kEsThreads) void expert_scan_kernel(int32_t* __restrict__ blk, int64_t nb, int E,
                                                                 int32_t* __restrict__ counts) {
  __shared__ int tot[kEsThreads / kWave];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t per = (nb + kEsThreads - 1) / kEsThreads;
  const int64_t b0 = min((int64_t)tid * per, nb), b1 = min(b0 + per, nb);
  int sum = 0;
  for (int64_t b = b0; b < b1; ++b) sum += blk[b * E + e];
  // exclusive scan of the per-thread sums across the workgroup, in thread order
  int x = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) tot[wave] = x;
  __syncthreads();
  int run = x - sum;
  for (int w = 0; w < wave; ++w) run += tot[w];
  for (int64_t b = b0; b < b1; ++b) {
    const int c = blk[b * E + e];
    blk[b * E + e] = run;
    run += c;
  }
  if (tid == kEsThreads - 1) counts[e] = run;
}

// Per block (one workgroup each, kScanThreads threads): thread e scans the kept
// loads min(counts[e], cap) into offsets (every workgroup does it for itself);
// then the block's assignments [b blen, (b + 1) blen) get their rows.  The first
// workgroup also writes offsets and the chunk lists.
__global__ __launch_bounds__(kScanThreads) void finalize_rows_kernel(
    const int32_t* __restrict__ idx, int64_t Tk, int k, int E, int64_t blen, int64_t cap,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ rank, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_of_slot, int32_t* __restrict__ token_of_row,
    Chunk* __restrict__ chunks, int32_t* __restrict__ n_chunks, ChunkCut cut, int64_t shared_rows,
    int64_t shared_row0) {
  __shared__ int tmp[kScanThreads];
  __shared__ int32_t offs[kMaxE];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  int load = 0;
  if (tid < E) {
    const int c = counts[tid];
    load = cap < 0 ? c : (int)min((int64_t)c, cap);
  }
  const int incl = block_inclusive_scan(load, tmp);
  const int excl = incl - load;
  if (tid < E) offs[tid] = excl;
  if (b == 0) {
    if (tid < E) offsets[tid] = excl;
    if (tid == E - 1) offsets[E] = incl;
    emit_chunks(tid < E, load, excl, E, cut, shared_rows, shared_row0, chunks, n_chunks, tmp);
  }
  __syncthreads();
  const int64_t begin = b * blen, end = min(begin + blen, Tk);
  for (int64_t i = begin + tid; i < end; i += kScanThreads) {
    const int e = idx[i];
    const int lr = rank[i];
    if (e < 0 || e >= E || lr < 0) {  // violated precondition: never index with it
      row_of_slot[i] = -1;
      continue;
    }
    const int64_t r = (int64_t)blk_base[b * E + e] + lr;
    if (cap < 0 || r < cap) {
      const int row = offs[e] + (int)r;
      row_of_slot[i] = row;
      token_of_row[row] = (int)(i / k);
    } else {
      row_of_slot[i] = -1;
    }
  }
}

// Small batches (T*k <= kScanThreads): rank, scan, chunk list and row maps in
// one workgroup of kScanThreads threads.  Wave 0 ranks the assignments as the
// block step does (one block); all threads then scan, cut the chunk list and
// write the row maps, with the ranks and offsets kept in LDS.
__device__ void dispatch_small_body(const int32_t* __restrict__ idx, int Tk, int k, int E, int64_t cap,
                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                    int32_t* __restrict__ row_of_slot, int32_t* __restrict__ token_of_row,
                                    Chunk* __restrict__ chunks, int32_t* __restrict__ n_chunks, const ChunkCut& cut,
                                    int64_t shared_rows, int64_t shared_row0) {
  __shared__ int32_t cnt[kMaxE];
  __shared__ int32_t offs[kMaxE];
  __shared__ int32_t rank_s[kScanThreads];
  __shared__ int tmp[kScanThreads];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kScanThreads) cnt[e] = 0;
  __syncthreads();
  if (tid < kWave)
    wave_rank([&](int64_t i) { return idx[i]; }, [&](int64_t i, int r) { rank_s[i] = r; }, Tk, E, cnt);
  __syncthreads();
  const int e = tid;
  int load = 0;
  if (e < E) {
    const int run = cnt[e];
    counts[e] = run;
    load = cap < 0 ? run : (int)min((int64_t)run, cap);
  }
  const int incl = block_inclusive_scan(load, tmp);
  const int excl = incl - load;
  if (e < E) {
    offsets[e] = excl;
    offs[e] = excl;
  }
  if (e == E - 1) offsets[E] = incl;
  emit_chunks(e < E, load, excl, E, cut, shared_rows, shared_row0, chunks, n_chunks, tmp);
  __syncthreads();
  if (tid < Tk) {
    const int r = rank_s[tid];
    const int ee = r < 0 ? -1 : idx[tid];
    if (r >= 0 && (cap < 0 || r < cap)) {
      const int row = offs[ee] + r;
      row_of_slot[tid] = row;
      token_of_row[row] = tid / k;
    } else {
      row_of_slot[tid] = -1;
    }
  }
}

__global__ __launch_bounds__(kScanThreads) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int Tk, int k, int E, int64_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_of_slot, int32_t* __restrict__ token_of_row,
    Chunk* __restrict__ chunks, int32_t* __restrict__ n_chunks, ChunkCut cut, int64_t shared_rows,
    int64_t shared_row0) {
  dispatch_small_body(idx, Tk, k, E, cap, counts, offsets, row_of_slot, token_of_row, chunks, n_chunks, cut,
                      shared_rows, shared_row0);
}

// ---- the router's select step (layer path, bf16) ----
// Partial logits part[s][t][0 .. Epad) of nsplit K slices (route.hip) are added
// in slice order (fixed, so the logits are reproducible), the logit bias is
// added, and one wave per token runs the gate and top-k (topk.h).

// zs[j][e] = sum over the nsplit slices, in slice order, of part[s][t0 + j][e]
// (+ bias[e]) for tokens j < nt and experts e < E.  Thread -> four consecutive
// experts of one token (16-byte loads; rows of Epad floats, a multiple of 32),
// every slice's load in flight at once (up to 8 slices per round).
__device__ __forceinline__ void sum_partials(const float* __restrict__ part, int nsplit, int T, int E, int t0, int nt,
                                             const float* __restrict__ bias, float* zs) {
  const int Epad = (E + 31) / 32 * 32, Q = Epad / 4;
  const int64_t stride4 = (int64_t)T * Epad / 4;
  for (int p = threadIdx.x; p < nt * Q; p += blockDim.x) {
    const int j = p / Q, qd = p - j * Q;
    const float4* pp = reinterpret_cast<const float4*>(part + (int64_t)(t0 + j) * Epad) + qd;
    float4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < nsplit; ks += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (ks + u < nsplit) v[u] = pp[(ks + u) * stride4];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (ks + u < nsplit) {
          sum.x += v[u].x;
          sum.y += v[u].y;
          sum.z += v[u].z;
          sum.w += v[u].w;
        }
    }
    const float sv[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = qd * 4 + c;
      if (e < E) zs[j * E + e] = bias != nullptr ? sv[c] + bias[e] : sv[c];
    }
  }
}

// Large batches: one workgroup = kSelTokens tokens, sixteen waves.  Thread
// (e, q) adds the partials of expert e for tokens q, q + 4, q + 8, q + 12 with
// every slice's load in flight at once (up to 8 slices per round), so the
// workgroup reads its partials in one or two round trips; wave j then runs the
// top-k of token j.  With blk != NULL it also runs the block step of the
// dispatch on its kSelTokens * k assignments (block b = this workgroup): local
// ranks into rank[], the block histogram into blk[b][0 .. E).
constexpr int kSelTokens = 16;
constexpr int kSelThreads = 1024;

template <int VPL>
__global__ __launch_bounds__(kSelThreads) void route_select_kernel(
    const float* __restrict__ part, int nsplit, int T, int E, const float* __restrict__ bias, int k, int gate,
    int renorm, float scale, RouteSel rs, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ blk, int32_t* __restrict__ rank) {
  // dynamic LDS: the summed logits [kSelTokens][E], then each wave's group scratch
  // [16][E] (only with expert groups)
  extern __shared__ __attribute__((aligned(16))) float sel_lds[];
  float* zs = sel_lds;
  float* wscr = sel_lds + kSelTokens * E;
  __shared__ int32_t cnt[kMaxE];
  __shared__ int32_t sel[kSelTokens * kMaxK];  // the block's selections, (token, slot) order
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kSelTokens;
  const int nt = min(kSelTokens, T - t0);
  for (int e = tid; e < E; e += kSelThreads) cnt[e] = 0;
  sum_partials(part, nsplit, T, E, t0, nt, bias, zs);
  __syncthreads();
  if (wave < nt) {
    const int t = t0 + wave;
    const SelOpts o{rs.sbias, rs.n_group, rs.topk_group, wscr + wave * E};
    float z[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + kWave * v;
      z[v] = e < E ? zs[wave * E + e] : -INFINITY;
    }
    topk_token<VPL>(z, E, k, gate, renorm, scale, o, rs.scores ? rs.scores + (int64_t)t * E : nullptr,
                    sel + wave * k, topk_w + (int64_t)t * k);
  }
  __syncthreads();
  const int64_t a0 = (int64_t)t0 * k;
  for (int i = tid; i < nt * k; i += kSelThreads) topk_idx[a0 + i] = sel[i];
  if (blk == nullptr) return;
  if (wave == 0)
    wave_rank([&](int64_t i) { return sel[i]; }, [&](int64_t i, int r) { rank[a0 + i] = r; }, (int64_t)nt * k, E,
              cnt);
  __syncthreads();
  for (int e = tid; e < E; e += kSelThreads) blk[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Small batches (T <= 16 tokens, T k <= kScanThreads assignments): one workgroup
// of kScanThreads threads adds the partials, runs the top-k of token t on wave
// t, then the whole dispatch (dispatch_small_body): routing and dispatch in one
// launch.
template <int VPL>
__global__ __launch_bounds__(kScanThreads) void route_select_small_kernel(
    const float* __restrict__ part, int nsplit, int T, int E, const float* __restrict__ bias, int k, int gate,
    int renorm, float scale, RouteSel rs, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int64_t cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_of_slot,
    int32_t* __restrict__ token_of_row, Chunk* __restrict__ chunks, int32_t* __restrict__ n_chunks, ChunkCut cut,
    int64_t shared_rows, int64_t shared_row0) {
  // dynamic LDS: the summed logits [T][E], then each wave's group scratch [16][E] (only with groups)
  extern __shared__ __attribute__((aligned(16))) float sel_lds[];
  float* zs = sel_lds;
  float* wscr = sel_lds + T * E;
  __shared__ int32_t sel[kGemvMaxT * kMaxK];  // the selections, (token, slot) order
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  sum_partials(part, nsplit, T, E, 0, T, bias, zs);
  __syncthreads();
  if (wave < T) {
    const SelOpts o{rs.sbias, rs.n_group, rs.topk_group, wscr + wave * E};
    float z[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + kWave * v;
      z[v] = e < E ? zs[wave * E + e] : -INFINITY;
    }
    topk_token<VPL>(z, E, k, gate, renorm, scale, o, rs.scores ? rs.scores + (int64_t)wave * E : nullptr,
                    sel + wave * k, topk_w + (int64_t)wave * k);
  }
  __syncthreads();
  for (int i = tid; i < T * k; i += kScanThreads) topk_idx[i] = sel[i];
  dispatch_small_body(sel, T * k, k, E, cap, counts, offsets, row_of_slot, token_of_row, chunks, n_chunks, cut,
                      shared_rows, shared_row0);
}

// Every one of the E groups holds C rows (row0 = e*C), then the shared rows.
__global__ __launch_bounds__(kScanThreads) void chunks_uniform_kernel(int E, int C, int64_t shared_rows,
                                                                      int64_t shared_row0, Chunk* __restrict__ chunks,
                                                                      int32_t* __restrict__ n_chunks, ChunkCut cut) {
  __shared__ int tmp[kScanThreads];
  const int e = threadIdx.x;
  emit_chunks(e < E, C, e * C, E, cut, shared_rows, shared_row0, chunks, n_chunks, tmp);
}
__global__ __launch_bounds__(kScanThreads) void chunks_from_offsets_kernel(
    const int32_t* __restrict__ offsets, int E, Chunk* __restrict__ chunks, int32_t* __restrict__ n_chunks,
    ChunkCut cut) {
  __shared__ int tmp[kScanThreads];
  const int e = threadIdx.x;
  const int row0 = e < E ? offsets[e] : 0;
  const int load = e < E ? offsets[e + 1] - row0 : 0;
  emit_chunks(e < E, load, row0, E, cut, 0, 0, chunks, n_chunks, tmp);
}

template <typename V>
__global__ __launch_bounds__(256) void gather_kernel(const V* __restrict__ x, const int32_t* __restrict__ tor,
                                                     const int32_t* __restrict__ offsets, int E,
                                                     int64_t rows_max, int64_t hv, V* __restrict__ xp) {
  const int64_t n = offsets[E];
  for (int64_t row = blockIdx.x; row < n && row < rows_max; row += gridDim.x) {
    const V* src = x + (int64_t)tor[row] * hv;
    V* dst = xp + row * hv;
    for (int64_t c = threadIdx.x; c < hv; c += blockDim.x) dst[c] = src[c];
  }
}

}  // namespace

// Blocks of the dispatch's block step: the stage entry point cuts the T*k
// assignments into hist_chunk() blocks, the layer's select kernel into blocks
// of kSelTokens tokens.
size_t dispatch_scratch_bytes(int64_t T, int64_t k, int64_t E) {
  const int64_t Tk = T * k;
  const int64_t nb = std::max<int64_t>(hist_blocks(Tk), (T + kSelTokens - 1) / kSelTokens);
  return align256((size_t)nb * E * 4) + align256((size_t)(Tk > 0 ? Tk : 1) * 4);
}

int64_t max_chunks(int64_t rows_max, int64_t E, int64_t shared_rows, int bm) {
  return E + (rows_max + bm - 1) / bm + (shared_rows + bm - 1) / bm + 1;
}

namespace {

struct DScratch {
  int32_t* blk;
  int32_t* rank;
};
DScratch dscratch_of(void* scratch, int64_t nb, int64_t E) {
  return DScratch{static_cast<int32_t*>(scratch),
                  reinterpret_cast<int32_t*>(static_cast<char*>(scratch) + align256((size_t)nb * E * 4))};
}

// Expert scan and finalize after a block step over nb blocks of blen assignments.
hipError_t launch_scan_finalize(int64_t T, int64_t k, int64_t E, int64_t cap, const int32_t* topk_idx,
                                const DScratch& d, int64_t nb, int64_t blen, int32_t* counts, int32_t* offsets,
                                int32_t* row_of_slot, int32_t* token_of_row, Chunk* chunks, int32_t* n_chunks,
                                const ChunkCut& cut, int64_t shared_rows, int64_t shared_row0, hipStream_t s) {
  hipLaunchKernelGGL(expert_scan_kernel, dim3((unsigned)E), dim3(kEsThreads), 0, s, d.blk, nb, (int)E, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(finalize_rows_kernel, dim3((unsigned)nb), dim3(kScanThreads), 0, s, topk_idx, T * k, (int)k,
                     (int)E, blen, cap, d.blk, d.rank, counts, offsets, row_of_slot, token_of_row, chunks, n_chunks,
                     cut, shared_rows, shared_row0);
  return hipGetLastError();
}

template <int VPL>
hipError_t select_t(const moe_config& c, const float* part, int nsplit, const float* bias, const RouteSel& rs,
                    int32_t* idx, float* tw, int32_t* blk, int32_t* rank, hipStream_t s) {
  const size_t lds = ((size_t)kSelTokens + (rs.n_group > 0 ? (size_t)kSelThreads / kWave : 0)) * c.E * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_select_kernel<VPL>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_kernel<VPL>, dim3((unsigned)((c.T + kSelTokens - 1) / kSelTokens)),
                     dim3(kSelThreads), lds, s, part, nsplit, (int)c.T, (int)c.E, bias, (int)c.k, c.gate,
                     c.renormalize, c.routed_scaling_factor, rs, idx, tw, blk, rank);
  return hipGetLastError();
}

hipError_t launch_select(const moe_config& c, const float* part, int nsplit, const float* bias, const RouteSel& rs,
                         int32_t* idx, float* tw, int32_t* blk, int32_t* rank, hipStream_t s) {
  if (c.E <= 64) return select_t<1>(c, part, nsplit, bias, rs, idx, tw, blk, rank, s);
  if (c.E <= 128) return select_t<2>(c, part, nsplit, bias, rs, idx, tw, blk, rank, s);
  if (c.E <= 256) return select_t<4>(c, part, nsplit, bias, rs, idx, tw, blk, rank, s);
  if (c.E <= 512) return select_t<8>(c, part, nsplit, bias, rs, idx, tw, blk, rank, s);
  return select_t<16>(c, part, nsplit, bias, rs, idx, tw, blk, rank, s);
}

template <int VPL>
hipError_t select_small_t(const moe_config& c, const float* part, int nsplit, const float* bias, const RouteSel& rs,
                          int32_t* idx, float* tw, int64_t cap, int32_t* counts, int32_t* offsets, int32_t* ros,
                          int32_t* tor, Chunk* chunks, int32_t* nch, const ChunkCut& cut, int64_t sh_rows,
                          int64_t sh_row0, hipStream_t s) {
  const size_t lds = ((size_t)c.T + (rs.n_group > 0 ? (size_t)kScanThreads / kWave : 0)) * c.E * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_select_small_kernel<VPL>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_select_small_kernel<VPL>, dim3(1), dim3(kScanThreads), lds, s, part, nsplit, (int)c.T,
                     (int)c.E, bias, (int)c.k, c.gate, c.renormalize, c.routed_scaling_factor, rs, idx, tw, cap, counts,
                     offsets, ros, tor, chunks, nch, cut, sh_rows, sh_row0);
  return hipGetLastError();
}

}  // namespace

bool route_dispatch_fused(const moe_config& c) { return c.dtype == MOE_BF16 && c.T <= kGemvMaxT; }

hipError_t launch_route_split(const moe_config& c, const void* x, const void* w, const float* bias,
                              const RouteSel& rs, int32_t* topk_idx, float* topk_w, void* scratch, hipStream_t s) {
  if (c.dtype != MOE_BF16) return launch_route(c, x, w, bias, rs, topk_idx, topk_w, s);
  float* part = static_cast<float*>(scratch);
  hipError_t e = launch_route_partials(c, x, w, part, s);
  if (e != hipSuccess) return e;
  return launch_select(c, part, route_partial_slices(c), bias, rs, topk_idx, topk_w, nullptr, nullptr, s);
}

hipError_t launch_route_dispatch(const moe_config& c, const void* x, const void* w, const float* bias,
                                 const RouteSel& rs, int32_t* topk_idx, float* topk_w, void* rscratch, int64_t cap,
                                 int32_t* counts, int32_t* offsets, int32_t* row_of_slot, int32_t* token_of_row,
                                 void* dscratch, Chunk* chunks, int32_t* n_chunks, const ChunkCut& cut,
                                 int64_t shared_rows, int64_t shared_row0, hipStream_t s,
                                 const std::function<hipError_t()>& routed) {
  float* part = static_cast<float*>(rscratch);
  const int nsplit = route_partial_slices(c);
  hipError_t e = launch_route_partials(c, x, w, part, s);
  if (e != hipSuccess) return e;
  if (route_dispatch_fused(c)) {
    const int E = (int)c.E;
#define MOE_SEL_SMALL(V)                                                                                        \
  select_small_t<V>(c, part, nsplit, bias, rs, topk_idx, topk_w, cap, counts, offsets, row_of_slot, token_of_row, \
                    chunks, n_chunks, cut, shared_rows, shared_row0, s)
    e = E <= 64 ? MOE_SEL_SMALL(1) : E <= 128 ? MOE_SEL_SMALL(2) : E <= 256 ? MOE_SEL_SMALL(4)
        : E <= 512 ? MOE_SEL_SMALL(8) : MOE_SEL_SMALL(16);
#undef MOE_SEL_SMALL
    if (e != hipSuccess) return e;
    return routed();
  }
  const int64_t nb = (c.T + kSelTokens - 1) / kSelTokens;
  const DScratch d = dscratch_of(dscratch, nb, c.E);
  e = launch_select(c, part, nsplit, bias, rs, topk_idx, topk_w, d.blk, d.rank, s);
  if (e != hipSuccess) return e;
  e = routed();
  if (e != hipSuccess) return e;
  return launch_scan_finalize(c.T, c.k, c.E, cap, topk_idx, d, nb, (int64_t)kSelTokens * c.k, counts, offsets,
                              row_of_slot, token_of_row, chunks, n_chunks, cut, shared_rows, shared_row0, s);
}

hipError_t launch_dispatch(int64_t T, int64_t k, int64_t E, int64_t cap, const int32_t* topk_idx,
                           int32_t* counts, int32_t* offsets, int32_t* row_of_slot,
                           int32_t* token_of_row, void* scratch, Chunk* chunks, int32_t* n_chunks,
                           const ChunkCut& cut, int64_t shared_rows, int64_t shared_row0, hipStream_t s) {
  const int64_t Tk = T * k;
  if (Tk <= kScanThreads) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kScanThreads), 0, s, topk_idx, (int)Tk, (int)k, (int)E,
                       cap, counts, offsets, row_of_slot, token_of_row, chunks, n_chunks, cut, shared_rows,
                       shared_row0);
    return hipGetLastError();
  }
  const int64_t ch = hist_chunk(Tk);
  const int64_t nb = hist_blocks(Tk);
  const DScratch d = dscratch_of(scratch, nb, E);
  hipLaunchKernelGGL(hist_rank_kernel, dim3((unsigned)nb), dim3(64), 0, s, topk_idx, Tk, (int)E, ch, d.blk, d.rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_scan_finalize(T, k, E, cap, topk_idx, d, nb, ch, counts, offsets, row_of_slot, token_of_row, chunks,
                              n_chunks, cut, shared_rows, shared_row0, s);
}

hipError_t launch_chunks_uniform(int64_t E, int64_t C, int64_t shared_rows, int64_t shared_row0, Chunk* chunks,
                                 int32_t* n_chunks, const ChunkCut& cut, hipStream_t s) {
  hipLaunchKernelGGL(chunks_uniform_kernel, dim3(1), dim3(kScanThreads), 0, s, (int)E, (int)C, shared_rows,
                     shared_row0, chunks, n_chunks, cut);
  return hipGetLastError();
}

hipError_t launch_chunks_from_offsets(const int32_t* offsets, int64_t E, Chunk* chunks, int32_t* n_chunks,
                                      const ChunkCut& cut, hipStream_t s) {
  hipLaunchKernelGGL(chunks_from_offsets_kernel, dim3(1), dim3(kScanThreads), 0, s, offsets, (int)E, chunks,
                     n_chunks, cut);
  return hipGetLastError();
}

hipError_t launch_gather(const void* x, const int32_t* token_of_row, const int32_t* offsets, int64_t E,
                         int64_t rows_max, int64_t H, int dtype, void* x_perm, hipStream_t s) {
  const int64_t bytes = H * (dtype == MOE_BF16 ? 2 : 4);
  const int64_t hv = bytes / 16;  // H is a multiple of 64: rows are whole 16-byte vectors
  const unsigned grid = (unsigned)std::min<int64_t>(std::max<int64_t>(rows_max, 1), 8192);
  hipLaunchKernelGGL(gather_kernel<uint4>, dim3(grid), dim3(256), 0, s, static_cast<const uint4*>(x),
                     token_of_row, offsets, (int)E, rows_max, hv, static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
