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
//   1. hist_rank   one wave per block of CH consecutive assignments walks them in
//                  order, 64 at a time; lanes with equal experts are grouped by a
//                  ballot match and ranked by lane order; a per-block LDS counter
//                  per expert carries the count across steps.  Emits the local rank
//                  and the block histogram.
//   2. scan        one workgroup: per expert, exclusive scan of the block histograms
//                  (block bases), demand counts, load = min(count, cap), offsets =
//                  exclusive scan of load, and the GEMM chunk list.
//   3. finalize    rank = block base + local rank; kept iff rank < cap;
//                  row_of_slot / token_of_row.
#include "common.h"

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

__global__ __launch_bounds__(64) void hist_rank_kernel(const int32_t* __restrict__ idx, int64_t Tk,
                                                       int E, int64_t CH, int32_t* __restrict__ blk_counts,
                                                       int32_t* __restrict__ rank_tmp) {
  __shared__ int32_t cnt[kMaxE];
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const int64_t begin = b * CH, end = min(begin + CH, Tk);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = begin; base < end; base += 64) {
    const int64_t i = base + lane;
    int e = i < end ? idx[i] : 0;
    const bool valid = i < end && e >= 0 && e < E;  // out-of-range ids (a violated precondition) are skipped
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bal = __ballot(valid && on);
      peers &= on ? bal : ~bal;
    }
    const int before = __popcll(peers & lt);
    const int old = valid ? cnt[e] : 0;
    __syncthreads();  // every lane has read its counter before the leaders update
    if (valid && before == 0) cnt[e] = old + __popcll(peers);
    if (valid) rank_tmp[i] = old + before;
    __syncthreads();
  }
  for (int e = lane; e < E; e += 64) blk_counts[b * E + e] = cnt[e];
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
  // the shared group follows its own cost, except that it never makes list B
  // on its own: a launch of only its few chunks would leave most CUs idle
  const bool sh_a = takes_list_a(shared_rows, cut) || total_b == 0;
  const int64_t sbm = sh_a ? cut.bm_a : cut.bm_b;
  const int nsh = (int)((shared_rows + sbm - 1) / sbm);
  const int sbase = sh_a ? total_a : total_b;
  Chunk* slist = sh_a ? chunks : chunks + cut.off_b;
  for (int c = tid; c < nsh; c += kScanThreads) {
    const int64_t r0 = c * shared_rows / nsh, r1 = (c + 1) * shared_rows / nsh;
    Chunk ck;
    ck.group = E;
    ck.row0 = (int)(shared_row0 + r0);
    ck.nrows = (int)(r1 - r0);
    ck.gfirst = sbase;
    ck.gcount = nsh;
    ck.pad[0] = ck.pad[1] = ck.pad[2] = 0;
    slist[sbase + c] = ck;
  }
  if (tid == 0) {
    n_chunks[0] = total_a + (sh_a ? nsh : 0);
    if (cut.bm_b != 0) n_chunks[1] = total_b + (sh_a ? 0 : nsh);
  }
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(
    int32_t* __restrict__ blk_counts, int64_t nb, int E, int64_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, Chunk* __restrict__ chunks, int32_t* __restrict__ n_chunks, ChunkCut cut,
    int64_t shared_rows, int64_t shared_row0) {
  __shared__ int tmp[kScanThreads];
  const int tid = threadIdx.x;
  const int e = tid;
  // exclusive block bases per expert, in block order: P threads per expert (thread q * E + e2 takes
  // blocks [q nb / P, (q + 1) nb / P) of expert e2), each summing its range, then rewriting it from
  // the sum of the ranges before it; sixteen independent loads per round
  const int P = max(1, kScanThreads / E);
  const int q = tid / E, e2 = tid - q * E;
  const bool part = q < P;
  const int64_t b0 = part ? q * nb / P : 0, b1 = part ? (q + 1) * nb / P : 0;
  int sum = 0;
  {
    int64_t b = b0;
    for (; b + 16 <= b1; b += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = blk_counts[(b + u) * E + e2];
#pragma unroll
      for (int u = 0; u < 16; ++u) sum += c[u];
    }
    for (; b < b1; ++b) sum += blk_counts[b * E + e2];
  }
  tmp[tid] = sum;
  __syncthreads();
  if (part) {
    int run = 0;
    for (int r = 0; r < q; ++r) run += tmp[r * E + e2];
    int64_t b = b0;
    for (; b + 16 <= b1; b += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = blk_counts[(b + u) * E + e2];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        blk_counts[(b + u) * E + e2] = run;
        run += c[u];
      }
    }
    for (; b < b1; ++b) {
      const int c = blk_counts[b * E + e2];
      blk_counts[b * E + e2] = run;
      run += c;
    }
  }
  int load = 0;
  if (e < E) {
    int run = 0;
    for (int r = 0; r < P; ++r) run += tmp[r * E + e];
    counts[e] = run;
    load = cap < 0 ? run : (int)min((int64_t)run, cap);
  }
  __syncthreads();  // tmp is reused by the scans below
  const int incl = block_inclusive_scan(load, tmp);
  const int excl = incl - load;
  if (e < E) offsets[e] = excl;
  if (e == E - 1) offsets[E] = incl;
  emit_chunks(e < E, load, excl, E, cut, shared_rows, shared_row0, chunks, n_chunks, tmp);
}

__global__ __launch_bounds__(256) void finalize_kernel(const int32_t* __restrict__ idx, int64_t Tk, int k,
                                                       int E, int64_t CH, int64_t cap,
                                                       const int32_t* __restrict__ blk_base,
                                                       const int32_t* __restrict__ rank_tmp,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ row_of_slot,
                                                       int32_t* __restrict__ token_of_row) {
  const int64_t b = blockIdx.x;
  const int64_t begin = b * CH, end = min(begin + CH, Tk);
  for (int64_t i = begin + threadIdx.x; i < end; i += blockDim.x) {
    const int e = idx[i];
    if (e < 0 || e >= E) {  // violated precondition: never index with it
      row_of_slot[i] = -1;
      continue;
    }
    const int64_t r = (int64_t)blk_base[b * E + e] + rank_tmp[i];
    if (cap < 0 || r < cap) {
      const int row = offsets[e] + (int)r;
      row_of_slot[i] = row;
      token_of_row[row] = (int)(i / k);
    } else {
      row_of_slot[i] = -1;
    }
  }
}

// Small batches (T*k <= kScanThreads): the three steps above in one workgroup.
// Wave 0 ranks the assignments exactly as hist_rank does (one block); all
// threads then scan, cut the chunk list and write the row maps, with the ranks
// and offsets kept in LDS.  Same outputs, one launch instead of three.
__global__ __launch_bounds__(kScanThreads) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int Tk, int k, int E, int64_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_of_slot, int32_t* __restrict__ token_of_row,
    Chunk* __restrict__ chunks, int32_t* __restrict__ n_chunks, ChunkCut cut, int64_t shared_rows,
    int64_t shared_row0) {
  __shared__ int32_t cnt[kMaxE];
  __shared__ int32_t offs[kMaxE];
  __shared__ int32_t rank_s[kScanThreads];
  __shared__ int tmp[kScanThreads];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int e = tid; e < E; e += kScanThreads) cnt[e] = 0;
  __syncthreads();
  if (tid < 64) {
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < Tk; base += 64) {
      const int i = base + lane;
      int e = i < Tk ? idx[i] : 0;
      const bool valid = i < Tk && e >= 0 && e < E;  // out-of-range ids (a violated precondition) are skipped
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
      if (i < Tk) rank_s[i] = valid ? old + before : -1;
      __builtin_amdgcn_wave_barrier();
    }
  }
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

size_t dispatch_scratch_bytes(int64_t Tk, int64_t E) {
  return align256((size_t)hist_blocks(Tk) * E * 4) + align256((size_t)(Tk > 0 ? Tk : 1) * 4);
}

int64_t max_chunks(int64_t rows_max, int64_t E, int64_t shared_rows, int bm) {
  return E + (rows_max + bm - 1) / bm + (shared_rows + bm - 1) / bm + 1;
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
  int32_t* blk = static_cast<int32_t*>(scratch);
  int32_t* rank_tmp = reinterpret_cast<int32_t*>(static_cast<char*>(scratch) + align256((size_t)nb * E * 4));
  hipLaunchKernelGGL(hist_rank_kernel, dim3((unsigned)nb), dim3(64), 0, s, topk_idx, Tk, (int)E, ch, blk,
                     rank_tmp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blk, nb, (int)E, cap, counts, offsets,
                     chunks, n_chunks, cut, shared_rows, shared_row0);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)nb), dim3(256), 0, s, topk_idx, Tk, (int)k, (int)E, ch,
                     cap, blk, rank_tmp, offsets, row_of_slot, token_of_row);
  return hipGetLastError();
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
