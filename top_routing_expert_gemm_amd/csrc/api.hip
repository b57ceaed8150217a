// C ABI of libmoe: host-side validation, workspace layout and launch sequence.
// The operations and their sources are documented in include/moe.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include "common.h"

using namespace moe;

namespace {

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline size_t esize(const moe_config* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

int64_t cap_of(const moe_config* c) {
  if (!(c->capacity_factor > 0.f)) return -1;
  const double v = ceil((double)c->capacity_factor * (double)c->T * (double)c->k / (double)c->E);
  return (int64_t)v;
}

// Device workspace of moe_forward; the stage entry points use the same layout.
struct Layout {
  size_t topk_idx, topk_w, counts, offsets, row_of_slot, token_of_row, dscratch, rscratch, chunks, n_chunks, h,
      y_perm, total;
  int64_t rows;    // permuted row space: T*k routed rows, then T shared rows
  ChunkPlan plan;  // chunk lists and their capacities
};

Layout layout(const moe_config* c) {
  Layout L;
  const int64_t Tk = c->T * c->k;
  const int64_t sh = c->n_shared ? c->T : 0;
  L.rows = Tk + sh;
  L.plan = chunk_plan(*c, Tk, sh, cap_of(c));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L.topk_idx = take((size_t)Tk * 4);
  L.topk_w = take((size_t)Tk * 4);
  L.counts = take((size_t)c->E * 4);
  L.offsets = take((size_t)(c->E + 1) * 4);
  L.row_of_slot = take((size_t)Tk * 4);
  L.token_of_row = take((size_t)Tk * 4);
  L.dscratch = take(dispatch_scratch_bytes(c->T, c->k, c->E));
  L.rscratch = take(route_scratch_bytes(*c));
  L.chunks = take((size_t)(L.plan.max_a + L.plan.max_b) * sizeof(Chunk));
  L.n_chunks = take(16);  // list sizes: gate/up A, B; down A, B
  L.h = take((size_t)L.rows * c->I * esize(c));
  L.y_perm = take((size_t)L.rows * c->H * esize(c));
  L.total = off;
  return L;
}

// Expert choice: C tokens per expert (capacity_factor <= 0 reads as 1), at most T.
int64_t ec_cap_of(const moe_config* c) {
  const double cf = c->capacity_factor > 0.f ? (double)c->capacity_factor : 1.0;
  const double v = ceil(cf * (double)c->T * (double)c->k / (double)c->E);
  return std::min<int64_t>(c->T, (int64_t)v);
}

// Device workspace of moe_forward_ec.
struct LayoutEC {
  size_t topk_idx, topk_w, scores, rscratch, token_of_row, row_of_pair, chunks, n_chunks, h, y_perm, total;
  int64_t C, rows;
  ChunkPlan plan;
};

LayoutEC layout_ec(const moe_config* c) {
  LayoutEC L;
  L.C = ec_cap_of(c);
  const int64_t R = c->E * L.C;
  const int64_t sh = c->n_shared ? c->T : 0;
  L.rows = R + sh;
  L.plan = chunk_plan(*c, R, sh, L.C);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L.topk_idx = take((size_t)c->T * c->k * 4);   // the router's own top-k, unused here
  L.topk_w = take((size_t)c->T * c->k * 4);
  L.scores = take((size_t)c->T * c->E * 4);
  L.rscratch = take(route_scratch_bytes(*c));
  L.token_of_row = take((size_t)R * 4);
  L.row_of_pair = take((size_t)c->T * c->E * 4);
  L.chunks = take((size_t)(L.plan.max_a + L.plan.max_b) * sizeof(Chunk));
  L.n_chunks = take(16);  // list sizes: gate/up A, B; down A, B
  L.h = take((size_t)L.rows * c->I * esize(c));
  L.y_perm = take((size_t)L.rows * c->H * esize(c));
  L.total = off;
  return L;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename P>
inline char* at(P* base, size_t off) {
  return static_cast<char*>(static_cast<void*>(base)) + off;
}

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

// Compute units of the current device (queried once per device; 0 if the query fails).
int device_cus() {
  constexpr int kDevs = 64;
  static std::once_flag once[kDevs];
  static int cus[kDevs];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 0;
  std::call_once(once[dev], [dev] {
    int v = 0;
    cus[dev] = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? v : 0;
  });
  return cus[dev];
}

// The chunk cut of plan p with what the dispatch step needs to place the shared
// group's gate/up chunks: the device's compute units and the gate/up pass's
// tiles per chunk (128 output columns each, gate and up side by side).
ChunkCut rounds_cut(const ChunkPlan& p, const moe_config* c) {
  ChunkCut cut = p.cut;
  cut.cus = device_cus();
  cut.nt = (int)((c->I + 127) / 128);
  return cut;
}

moe_status check_ws(const moe_config* c, void* ws, size_t ws_bytes) {
  if (ws == nullptr) return MOE_ERR_WORKSPACE;
  if (ws_bytes < layout(c).total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

#define MOE_TRY(expr)                          \
  do {                                         \
    moe_status _s = (expr);                    \
    if (_s != MOE_OK) return _s;               \
  } while (0)
#define HIP_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

moe_status need(const void* p) { return p == nullptr ? MOE_ERR_NULL : (aligned16(p) ? MOE_OK : MOE_ERR_ALIGN); }
moe_status opt(const void* p) { return p == nullptr || aligned16(p) ? MOE_OK : MOE_ERR_ALIGN; }


// One grouped-GEMM pass over the chunk lists of plan p: launch(g) with g on
// list A, then on list B when the plan has one.
template <typename F>
hipError_t each_list(GemmArgs g, const ChunkPlan& p, Chunk* chunks, int32_t* nch, F launch) {
  g.chunks = chunks;
  g.n_chunks = nch;
  g.max_chunks = p.max_a;
  g.bm = p.cut.bm_a;
  const hipError_t e = launch(g);
  if (e != hipSuccess || p.cut.bm_b == 0) return e;
  g.chunks = chunks + p.cut.off_b;
  g.n_chunks = nch + 1;
  g.max_chunks = p.max_b;
  g.bm = p.cut.bm_b;
  return launch(g);
}

// The down pass (bf16 or fp32 weights) over the chunk lists of plan p (nch:
// the down pass's two list sizes, which place the shared group's chunks): both
// lists in one launch where the 320-row kernel takes the pass, else each list
// on its own launch.
hipError_t down_lists(GemmArgs g, const ChunkPlan& p, Chunk* chunks, int32_t* nch, int dtype, hipStream_t s) {
  if (p.cut.bm_b != 0) {
    GemmArgs b = g;
    b.chunks = chunks;
    b.n_chunks = nch;
    b.chunks_b = chunks + p.cut.off_b;
    b.n_chunks_b = nch + 1;
    b.max_chunks = p.max_a + p.max_b;
    b.bm = kGemmBMdl;
    hipError_t e = hipSuccess;
    if (launch_down_both(b, dtype, s, e)) return e;
  }
  return each_list(g, p, chunks, nch, [&](const GemmArgs& a) { return launch_down(a, dtype, s); });
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "shape outside the supported range";
    case MOE_ERR_UNSUPPORTED: return "unsupported option";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MOE_ERR_SCRATCH: return "layer needs more workspace than the static device scratch holds";
  }
  return "unknown status";
}

moe_status moe_validate(const moe_config* c) {
  if (c == nullptr) return MOE_ERR_NULL;
  if (c->T < 1 || c->E < 1 || c->E > kMaxE || c->k < 1 || c->k > kMaxK || c->k > c->E) return MOE_ERR_SHAPE;
  if (c->H < 64 || c->H % 64 != 0 || c->I < 64 || c->I % 64 != 0) return MOE_ERR_SHAPE;
  if (c->gate != MOE_GATE_SOFTMAX && c->gate != MOE_GATE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_SHAPE;
  if (!isfinite(c->routed_scaling_factor) || !isfinite(c->capacity_factor)) return MOE_ERR_SHAPE;
  if (c->n_shared < 0 || c->n_shared > 1) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared == 1 && c->I_shared != c->I) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = c->T * c->k + c->T;
  if (c->T > (int64_t(1) << 31) || rows >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (c->H > (int64_t(1) << 20) || c->I > (int64_t(1) << 20)) return MOE_ERR_SHAPE;
  if (c->n_group < 0 || c->n_group > 64) return MOE_ERR_SHAPE;
  if (c->n_group > 0) {
    if (c->E % c->n_group != 0 || c->topk_group < 1 || c->topk_group > c->n_group) return MOE_ERR_SHAPE;
    if (c->k > (int64_t)c->topk_group * (c->E / c->n_group)) return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_config* c, size_t* bytes) {
  MOE_TRY(moe_validate(c));
  if (bytes == nullptr) return MOE_ERR_NULL;
  *bytes = layout(c).total;
  return MOE_OK;
}

int64_t moe_capacity(const moe_config* c) {
  if (moe_validate(c) != MOE_OK) return -1;
  return cap_of(c);
}

moe_status moe_layer_params(const moe_config* c, int64_t* total, int64_t* active) {
  MOE_TRY(moe_validate(c));
  if (total == nullptr || active == nullptr) return MOE_ERR_NULL;
  const int64_t per_expert = 3 * c->H * c->I;
  const int64_t router = c->E * c->H;
  const int64_t shared = c->n_shared * 3 * c->H * c->I_shared;
  *total = c->E * per_expert + router + shared;
  *active = c->k * per_expert + router + shared;
  return MOE_OK;
}

moe_status moe_route_sel(const moe_config* c, const void* x, const void* w_router, const float* router_bias,
                         const float* score_bias, int32_t* topk_idx, float* topk_w, float* scores,
                         void* stream) {
  MOE_TRY(moe_validate(c));
  MOE_TRY(need(x));
  MOE_TRY(need(w_router));
  MOE_TRY(need(topk_idx));
  MOE_TRY(need(topk_w));
  MOE_TRY(opt(router_bias));
  MOE_TRY(opt(score_bias));
  MOE_TRY(opt(scores));
  HIP_TRY(launch_route(*c, x, w_router, router_bias, route_sel_of(*c, score_bias, scores), topk_idx, topk_w,
                       S(stream)));
  return MOE_OK;
}

moe_status moe_route(const moe_config* c, const void* x, const void* w_router, const float* router_bias,
                     int32_t* topk_idx, float* topk_w, void* stream) {
  return moe_route_sel(c, x, w_router, router_bias, nullptr, topk_idx, topk_w, nullptr, stream);
}

moe_status moe_balance_stats(const moe_config* c, const int32_t* counts, const float* scores, float* score_mean,
                             float* load_frac, float* balance, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(moe_validate(c));
  MOE_TRY(need(counts));
  MOE_TRY(need(scores));
  MOE_TRY(opt(score_mean));
  MOE_TRY(opt(load_frac));
  MOE_TRY(opt(balance));
  if (ws == nullptr || ws_bytes < stats_scratch_bytes(*c)) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  HIP_TRY(launch_balance_stats(*c, counts, scores, score_mean, load_frac, balance, ws, S(stream)));
  return MOE_OK;
}

moe_status moe_bias_update(const moe_config* c, const int32_t* counts, float gamma, float* score_bias,
                           void* stream) {
  MOE_TRY(moe_validate(c));
  MOE_TRY(need(counts));
  MOE_TRY(need(score_bias));
  if (!isfinite(gamma)) return MOE_ERR_SHAPE;
  HIP_TRY(launch_bias_update(*c, counts, gamma, score_bias, S(stream)));
  return MOE_OK;
}

moe_status moe_dispatch(const moe_config* c, const int32_t* topk_idx, const void* x, int32_t* counts,
                        int32_t* offsets, int32_t* row_of_slot, int32_t* token_of_row, void* x_perm, void* ws,
                        size_t ws_bytes, void* stream) {
  MOE_TRY(moe_validate(c));
  MOE_TRY(need(topk_idx));
  MOE_TRY(need(counts));
  MOE_TRY(need(offsets));
  MOE_TRY(need(row_of_slot));
  MOE_TRY(need(token_of_row));
  MOE_TRY(opt(x_perm));
  if (x_perm != nullptr) MOE_TRY(need(x));
  MOE_TRY(check_ws(c, ws, ws_bytes));
  const Layout L = layout(c);
  HIP_TRY(launch_dispatch(c->T, c->k, c->E, cap_of(c), topk_idx, counts, offsets, row_of_slot, token_of_row,
                          at(ws, L.dscratch), reinterpret_cast<Chunk*>(at(ws, L.chunks)),
                          reinterpret_cast<int32_t*>(at(ws, L.n_chunks)), rounds_cut(L.plan, c), 0, 0, S(stream)));
  if (x_perm != nullptr)
    HIP_TRY(launch_gather(x, token_of_row, offsets, c->E, c->T * c->k, c->H, c->dtype, x_perm, S(stream)));
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config* c, const void* x_perm, const int32_t* offsets, const void* w_gate,
                          const void* w_up, const void* w_down, void* y_perm, void* ws, size_t ws_bytes,
                          void* stream) {
  MOE_TRY(moe_validate(c));
  MOE_TRY(need(x_perm));
  MOE_TRY(need(offsets));
  MOE_TRY(need(w_gate));
  MOE_TRY(need(w_up));
  MOE_TRY(need(w_down));
  MOE_TRY(need(y_perm));
  MOE_TRY(check_ws(c, ws, ws_bytes));
  const Layout L = layout(c);
  Chunk* chunks = reinterpret_cast<Chunk*>(at(ws, L.chunks));
  int32_t* nch = reinterpret_cast<int32_t*>(at(ws, L.n_chunks));
  hipStream_t s = S(stream);
  HIP_TRY(launch_chunks_from_offsets(offsets, c->E, chunks, nch, L.plan.cut, s));
  GemmArgs g{};
  g.A = x_perm;
  g.gather = nullptr;
  g.shared_row0 = 0;
  g.w0 = w_gate;
  g.w1 = w_up;
  g.E = c->E;
  g.K = c->H;
  g.N = c->I;
  g.a_rows = c->T * c->k;
  g.out = at(ws, L.h);
  HIP_TRY(each_list(g, L.plan, chunks, nch, [&](const GemmArgs& a) { return launch_gateup(a, c->dtype, s); }));
  g.A = at(ws, L.h);
  g.w0 = w_down;
  g.w1 = nullptr;
  g.K = c->I;
  g.N = c->H;
  g.out = y_perm;
  HIP_TRY(down_lists(g, L.plan, chunks, nch + 2, c->dtype, s));
  return MOE_OK;
}

moe_status moe_combine(const moe_config* c, const void* y_perm, const int32_t* row_of_slot, const float* topk_w,
                       const void* y_shared, void* y, void* stream) {
  MOE_TRY(moe_validate(c));
  MOE_TRY(need(y_perm));
  MOE_TRY(need(row_of_slot));
  MOE_TRY(need(topk_w));
  MOE_TRY(opt(y_shared));
  MOE_TRY(need(y));
  HIP_TRY(launch_combine(y_perm, row_of_slot, topk_w, y_shared, y, c->T, c->H, c->k, c->dtype, S(stream)));
  return MOE_OK;
}

// The layer's stage sequence; expert weights from `w` (cfg->dtype) or, when q is
// not NULL, from the FP8 experts of q (decode batches only, checked by the caller).
static moe_status forward_impl(const moe_config* c, const moe_weights* w, const moe_fp8_experts* q, const void* x,
                               void* y, moe_route_out* ro, void* ws, size_t ws_bytes, void* stream,
                               void* const* events) {
  MOE_TRY(moe_validate(c));
  if (w == nullptr) return MOE_ERR_NULL;
  MOE_TRY(need(x));
  MOE_TRY(need(y));
  MOE_TRY(need(w->w_router));
  MOE_TRY(opt(w->router_bias));
  MOE_TRY(opt(w->score_bias));
  if (q == nullptr) {
    MOE_TRY(need(w->w_gate));
    MOE_TRY(need(w->w_up));
    MOE_TRY(need(w->w_down));
    if (c->n_shared) {
      MOE_TRY(need(w->ws_gate));
      MOE_TRY(need(w->ws_up));
      MOE_TRY(need(w->ws_down));
    }
  } else {
    MOE_TRY(need(q->w_gate));
    MOE_TRY(need(q->w_up));
    MOE_TRY(need(q->w_down));
    MOE_TRY(need(q->s_gate));
    MOE_TRY(need(q->s_up));
    MOE_TRY(need(q->s_down));
    if (c->n_shared) {
      MOE_TRY(need(q->ws_gate));
      MOE_TRY(need(q->ws_up));
      MOE_TRY(need(q->ws_down));
      MOE_TRY(need(q->ss_gate));
      MOE_TRY(need(q->ss_up));
      MOE_TRY(need(q->ss_down));
    }
  }
  MOE_TRY(check_ws(c, ws, ws_bytes));
  const Layout L = layout(c);
  moe_route_out r{};
  if (ro != nullptr) r = *ro;
  if (r.topk_idx == nullptr) r.topk_idx = reinterpret_cast<int32_t*>(at(ws, L.topk_idx));
  if (r.topk_w == nullptr) r.topk_w = reinterpret_cast<float*>(at(ws, L.topk_w));
  if (r.counts == nullptr) r.counts = reinterpret_cast<int32_t*>(at(ws, L.counts));
  if (r.offsets == nullptr) r.offsets = reinterpret_cast<int32_t*>(at(ws, L.offsets));
  if (r.row_of_slot == nullptr) r.row_of_slot = reinterpret_cast<int32_t*>(at(ws, L.row_of_slot));
  if (r.token_of_row == nullptr) r.token_of_row = reinterpret_cast<int32_t*>(at(ws, L.token_of_row));
  MOE_TRY(need(r.topk_idx));
  MOE_TRY(need(r.topk_w));
  MOE_TRY(need(r.counts));
  MOE_TRY(need(r.offsets));
  MOE_TRY(need(r.row_of_slot));
  MOE_TRY(need(r.token_of_row));
  MOE_TRY(opt(r.scores));

  hipStream_t s = S(stream);
  auto mark = [&](int i) -> hipError_t {
    if (events == nullptr || events[i] == nullptr) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
  };
  const int64_t Tk = c->T * c->k;
  const int64_t sh = c->n_shared ? c->T : 0;
  Chunk* chunks = reinterpret_cast<Chunk*>(at(ws, L.chunks));
  int32_t* nch = reinterpret_cast<int32_t*>(at(ws, L.n_chunks));

  HIP_TRY(mark(0));
  if (c->dtype == MOE_BF16) {
    HIP_TRY(launch_route_dispatch(*c, x, w->w_router, w->router_bias, route_sel_of(*c, w->score_bias, r.scores),
                                  r.topk_idx, r.topk_w, at(ws, L.rscratch), cap_of(c), r.counts, r.offsets,
                                  r.row_of_slot, r.token_of_row, at(ws, L.dscratch), chunks, nch, rounds_cut(L.plan, c), sh, Tk,
                                  s, [&] { return mark(1); }));
  } else {
    HIP_TRY(launch_route(*c, x, w->w_router, w->router_bias, route_sel_of(*c, w->score_bias, r.scores),
                         r.topk_idx, r.topk_w, s));
    HIP_TRY(mark(1));
    HIP_TRY(launch_dispatch(c->T, c->k, c->E, cap_of(c), r.topk_idx, r.counts, r.offsets, r.row_of_slot,
                            r.token_of_row, at(ws, L.dscratch), chunks, nch, rounds_cut(L.plan, c), sh, Tk, s));
  }
  HIP_TRY(mark(2));
  GemmArgs g{};
  g.A = x;
  g.gather = r.token_of_row;
  g.shared_row0 = Tk;
  if (q == nullptr) {
    g.w0 = w->w_gate;
    g.w1 = w->w_up;
    g.ws0 = w->ws_gate;
    g.ws1 = w->ws_up;
  } else {
    g.w0 = q->w_gate;
    g.w1 = q->w_up;
    g.ws0 = q->ws_gate;
    g.ws1 = q->ws_up;
    g.sc0 = q->s_gate;
    g.sc1 = q->s_up;
    g.ssc0 = q->ss_gate;
    g.ssc1 = q->ss_up;
  }
  g.E = c->E;
  g.K = c->H;
  g.N = c->I;
  g.a_rows = c->T;
  g.out = at(ws, L.h);
  g.nt_out = true;
  HIP_TRY(each_list(g, L.plan, chunks, nch, [&](const GemmArgs& a) {
    return q == nullptr ? launch_gateup(a, c->dtype, s) : launch_gateup_fp8(a, s);
  }));
  HIP_TRY(mark(3));
  g.A = at(ws, L.h);
  g.gather = nullptr;
  if (q == nullptr) {
    g.w0 = w->w_down;
    g.ws0 = w->ws_down;
  } else {
    g.w0 = q->w_down;
    g.ws0 = q->ws_down;
    g.sc0 = q->s_down;
    g.ssc0 = q->ss_down;
    g.sc1 = g.ssc1 = nullptr;
  }
  g.w1 = nullptr;
  g.ws1 = nullptr;
  g.K = c->I;
  g.N = c->H;
  g.a_rows = L.rows;
  g.out = at(ws, L.y_perm);
  g.nt_out = (int64_t)L.rows * c->H * (int64_t)esize(c) > kLastLevelCacheBytes;
  if (q == nullptr)
    HIP_TRY(down_lists(g, L.plan, chunks, nch + 2, c->dtype, s));
  else
    HIP_TRY(each_list(g, L.plan, chunks, nch + 2, [&](const GemmArgs& a) { return launch_down_fp8(a, s); }));
  HIP_TRY(mark(4));
  const void* ysh = c->n_shared ? static_cast<const void*>(at(ws, L.y_perm + (size_t)Tk * c->H * esize(c))) : nullptr;
  HIP_TRY(launch_combine(at(ws, L.y_perm), r.row_of_slot, r.topk_w, ysh, y, c->T, c->H, c->k, c->dtype, s));
  HIP_TRY(mark(5));
  return MOE_OK;
}

moe_status moe_forward_timed(const moe_config* c, const moe_weights* w, const void* x, void* y,
                             moe_route_out* ro, void* ws, size_t ws_bytes, void* stream, void* const* events) {
  return forward_impl(c, w, nullptr, x, y, ro, ws, ws_bytes, stream, events);
}

moe_status moe_forward(const moe_config* c, const moe_weights* w, const void* x, void* y, moe_route_out* ro,
                       void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(c, w, nullptr, x, y, ro, ws, ws_bytes, stream, nullptr);
}

}  // extern "C"

// ---- moe_forward without allocation: a static device scratch per GPU ----
// The workspace lives in a file-scope device array.  On the host its name is
// only a stand-in for the symbol: the device address of each GPU's copy comes
// from hipGetSymbolAddress with that GPU current, taken once per device and
// kept; kernels and copies get that address, never the array's name.
namespace {
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch, or nullptr on failure.
void* static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot& sl = g_scratch[dev];
  std::call_once(sl.once, [&sl] { sl.err = hipGetSymbolAddress(&sl.ptr, HIP_SYMBOL(scratch)); });
  return sl.err == hipSuccess ? sl.ptr : nullptr;
}
}  // namespace

extern "C" {

size_t moe_static_scratch_bytes(void) { return MOE_STATIC_SCRATCH_BYTES; }

moe_status moe_forward_noalloc(const moe_config* c, const moe_weights* w, const void* x, void* y,
                               moe_route_out* ro, void* stream) {
  MOE_TRY(moe_validate(c));
  if (layout(c).total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = static_scratch();
  if (ws == nullptr) return MOE_ERR_HIP;
  // every stage writes what a later one reads (no counter or flag starts from a
  // cleared value), so the scratch is not cleared between calls
  return forward_impl(c, w, nullptr, x, y, ro, ws, MOE_STATIC_SCRATCH_BYTES, stream, nullptr);
}

// ---- FP8 expert weights ----

moe_status moe_quantize_fp8(const void* w, int32_t dtype, int64_t G, int64_t N, int64_t K, uint8_t* codes,
                            float* scales, void* stream) {
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (G < 1 || N < kFp8Block || K < kFp8Block || N % kFp8Block != 0 || K % kFp8Block != 0) return MOE_ERR_SHAPE;
  if (G > 65535 || (N / kFp8Block) * (K / kFp8Block) > (int64_t(1) << 31) - 1) return MOE_ERR_SHAPE;
  MOE_TRY(need(w));
  MOE_TRY(need(codes));
  MOE_TRY(need(scales));
  HIP_TRY(launch_quantize_fp8(w, dtype, G, N, K, codes, scales, S(stream)));
  return MOE_OK;
}

moe_status moe_mfma_peak(int64_t iters, int32_t varied, float* sink, int64_t* flops, void* stream) {
  if (iters < 1 || iters > (int64_t(1) << 24) || (varied != 0 && varied != 1)) return MOE_ERR_SHAPE;
  if (flops == nullptr) return MOE_ERR_NULL;
  MOE_TRY(need(sink));
  *flops = mfma_peak_flops(iters);
  HIP_TRY(launch_mfma_peak((int)iters, varied != 0, sink, S(stream)));
  return MOE_OK;
}

moe_status moe_hbm_read_peak(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < kReadBlockBytes || bytes % kReadBlockBytes != 0 || bytes > (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  MOE_TRY(need(buf));
  MOE_TRY(need(sink));
  HIP_TRY(launch_hbm_read(buf, bytes / kReadBlockBytes, sink, S(stream)));
  return MOE_OK;
}

moe_status moe_forward_fp8(const moe_config* c, const moe_weights* w, const moe_fp8_experts* q, const void* x,
                           void* y, moe_route_out* ro, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(moe_validate(c));
  if (q == nullptr) return MOE_ERR_NULL;
  if (c->dtype != MOE_BF16 || c->T > kGemvMaxT) return MOE_ERR_UNSUPPORTED;
  if (c->H % kFp8Block != 0 || c->I % kFp8Block != 0) return MOE_ERR_SHAPE;
  return forward_impl(c, w, q, x, y, ro, ws, ws_bytes, stream, nullptr);
}

// ---- expert choice ----

static moe_status validate_ec(const moe_config* c) {
  MOE_TRY(moe_validate(c));
  const int64_t C = ec_cap_of(c);
  if (c->E * C + c->T >= (int64_t(1) << 31) || c->T * c->E >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

int64_t moe_ec_capacity(const moe_config* c) {
  if (validate_ec(c) != MOE_OK) return -1;
  return ec_cap_of(c);
}

moe_status moe_ec_workspace_size(const moe_config* c, size_t* bytes) {
  MOE_TRY(validate_ec(c));
  if (bytes == nullptr) return MOE_ERR_NULL;
  *bytes = layout_ec(c).total;
  return MOE_OK;
}

moe_status moe_route_ec(const moe_config* c, const float* scores, int32_t* token_of_row, int32_t* row_of_pair,
                        void* stream) {
  MOE_TRY(validate_ec(c));
  MOE_TRY(need(scores));
  MOE_TRY(need(token_of_row));
  MOE_TRY(need(row_of_pair));
  HIP_TRY(launch_ec_select(scores, c->T, c->E, ec_cap_of(c), token_of_row, row_of_pair, S(stream)));
  return MOE_OK;
}

moe_status moe_forward_ec(const moe_config* c, const moe_weights* w, const void* x, void* y, moe_ec_out* eo,
                          void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate_ec(c));
  if (w == nullptr) return MOE_ERR_NULL;
  MOE_TRY(need(x));
  MOE_TRY(need(y));
  MOE_TRY(need(w->w_router));
  MOE_TRY(opt(w->router_bias));
  MOE_TRY(need(w->w_gate));
  MOE_TRY(need(w->w_up));
  MOE_TRY(need(w->w_down));
  if (c->n_shared) {
    MOE_TRY(need(w->ws_gate));
    MOE_TRY(need(w->ws_up));
    MOE_TRY(need(w->ws_down));
  }
  const LayoutEC L = layout_ec(c);
  if (ws == nullptr || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  moe_ec_out o{};
  if (eo != nullptr) o = *eo;
  if (o.scores == nullptr) o.scores = reinterpret_cast<float*>(at(ws, L.scores));
  if (o.token_of_row == nullptr) o.token_of_row = reinterpret_cast<int32_t*>(at(ws, L.token_of_row));
  if (o.row_of_pair == nullptr) o.row_of_pair = reinterpret_cast<int32_t*>(at(ws, L.row_of_pair));
  MOE_TRY(need(o.scores));
  MOE_TRY(need(o.token_of_row));
  MOE_TRY(need(o.row_of_pair));

  hipStream_t s = S(stream);
  const int64_t R = c->E * L.C;
  const int64_t sh = c->n_shared ? c->T : 0;
  Chunk* chunks = reinterpret_cast<Chunk*>(at(ws, L.chunks));
  int32_t* nch = reinterpret_cast<int32_t*>(at(ws, L.n_chunks));
  // router + gate (its top-k output is not used), then the per-expert top-C
  HIP_TRY(launch_route_split(*c, x, w->w_router, w->router_bias, RouteSel{nullptr, 0, 0, o.scores},
                             reinterpret_cast<int32_t*>(at(ws, L.topk_idx)), reinterpret_cast<float*>(at(ws, L.topk_w)),
                             at(ws, L.rscratch), s));
  HIP_TRY(launch_ec_select(o.scores, c->T, c->E, L.C, o.token_of_row, o.row_of_pair, s));
  HIP_TRY(launch_chunks_uniform(c->E, L.C, sh, R, chunks, nch, rounds_cut(L.plan, c), s));
  GemmArgs g{};
  g.A = x;
  g.gather = o.token_of_row;
  g.shared_row0 = R;
  g.w0 = w->w_gate;
  g.w1 = w->w_up;
  g.ws0 = w->ws_gate;
  g.ws1 = w->ws_up;
  g.E = c->E;
  g.K = c->H;
  g.N = c->I;
  g.a_rows = c->T;
  g.out = at(ws, L.h);
  g.nt_out = true;
  HIP_TRY(each_list(g, L.plan, chunks, nch, [&](const GemmArgs& a) { return launch_gateup(a, c->dtype, s); }));
  g.A = at(ws, L.h);
  g.gather = nullptr;
  g.w0 = w->w_down;
  g.w1 = nullptr;
  g.ws0 = w->ws_down;
  g.ws1 = nullptr;
  g.K = c->I;
  g.N = c->H;
  g.a_rows = L.rows;
  g.out = at(ws, L.y_perm);
  g.nt_out = (int64_t)L.rows * c->H * (int64_t)esize(c) > kLastLevelCacheBytes;
  HIP_TRY(down_lists(g, L.plan, chunks, nch + 2, c->dtype, s));
  const void* ysh = c->n_shared ? static_cast<const void*>(at(ws, L.y_perm + (size_t)R * c->H * esize(c))) : nullptr;
  // weight of a chosen pair: its gate score times routed_scaling_factor
  HIP_TRY(launch_combine(at(ws, L.y_perm), o.row_of_pair, o.scores, ysh, y, c->T, c->H, c->E, c->dtype, s,
                         c->routed_scaling_factor));
  return MOE_OK;
}

}  // extern "C"
