// Host side of libmoedet: argument validation, workspace planning and the
// launch sequence of each C-ABI call (declared in include/moedet.h).
//
// Work decompositions that depend on routing (rows per expert, split-K
// chunks) are derived on the device from counts[]; the host sizes grids and
// workspaces from shape upper bounds only, so nothing here waits for the GPU.
#include <string.h>

#include <mutex>

#include "../../include/moedet.h"
#include "kernels.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moedet {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  bool bf16;
  int64_t T;
  int D, F, E, k, eb, el;
  int64_t rows_cap;
  int64_t nslot;      // T*k
  int nchunk;         // routing chunks
  int bm, bn;         // GEMM tile
  int n_tiles;        // fc2-dgrad N-tiles (dprob partials per row)
  int kc;             // wgrad K chunk (rows)
  bool may_split;     // some expert can hold more than kc rows
  int64_t wslots;     // wgrad partial slots per dW
  int64_t mt_cap;     // routing.sched: row-tile entries (bm rows)
  int64_t wu_cap;     // routing.sched: weight-gradient unit entries
  int bm2;            // height of the second row-tile list
  int64_t mt_cap2;    // routing.sched: row-tile entries (bm2 rows)
  int64_t list2_at;   // routing.sched: int32 offset of the bm2 list
  int64_t aux_at;     // routing.sched: int32 offset of the unit side table
  int64_t pad_at;     // routing.sched: int32 offset of the padded row offsets
  int64_t rpad_cap;   // MXFP8 weight-gradient operands: padded rows (bytes per codes row)
  bool fc1_list2;     // the fc1 dgrad runs the bm2 list
  int64_t sched_elems;
  size_t esize;
};

moe_status validate(const moe_problem* p, Plan* pl) {
  if (!p) return MOE_ERR_NULL;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (p->combine != 0 && p->combine != 1) return MOE_ERR_MODE;
  if (p->tokens < 0 || p->tokens >= (int64_t)1 << 31) return MOE_ERR_SHAPE;
  if (p->num_experts < 1 || p->num_experts > kMaxExperts) return MOE_ERR_SHAPE;
  if (p->top_k < 1 || p->top_k > p->num_experts || p->top_k > kMaxTopK) return MOE_ERR_SHAPE;
  if (p->expert_begin < 0 || p->num_local < 1 || p->expert_begin + p->num_local > p->num_experts)
    return MOE_ERR_SHAPE;
  if (p->combine == 1 && (p->expert_begin != 0 || p->num_local != p->num_experts)) return MOE_ERR_SHAPE;
  if (p->tokens * p->top_k >= (int64_t)1 << 31) return MOE_ERR_SHAPE;
  const bool bf16 = p->dtype == MOE_BF16;
  const int bm = gemm_tile_m(bf16), bn = gemm_tile_n(bf16);
  const int align = bf16 ? 256 : 64;
  if (p->d_model <= 0 || p->d_ffn <= 0 || p->d_model % align || p->d_ffn % align) return MOE_ERR_SHAPE;
  if (p->d_ffn / bn > 64) return MOE_ERR_SHAPE;  // dprob partials per row
  if ((int64_t)p->d_model * p->d_ffn >= (int64_t)1 << 31) return MOE_ERR_SHAPE;
  {
    // Token arrays ([T, D]: x, dy, y, dx) are gathered through 32-bit buffer
    // offsets and stay below 2 GiB; arrays of routed rows ([rows_cap,
    // max(D, F)]) are addressed from each tile's first row and may reach
    // 32 GiB (so the act_p prologue's 16-byte vectors number below 2^31).
    const int64_t es = bf16 ? 2 : 4;
    const int64_t rc = p->tokens * (int64_t)(p->top_k < p->num_local ? p->top_k : p->num_local);
    const int64_t wmax = p->d_model > p->d_ffn ? p->d_model : p->d_ffn;
    if (p->tokens * p->d_model * es >= ((int64_t)1 << 31) || rc * wmax * es >= ((int64_t)1 << 35))
      return MOE_ERR_SHAPE;
  }
  if (p->n_stage_events < 0 || (p->n_stage_events > 0 && !p->stage_events)) return MOE_ERR_NULL;
  if (pl) {
    pl->bf16 = bf16;
    pl->T = p->tokens;
    pl->D = p->d_model;
    pl->F = p->d_ffn;
    pl->E = p->num_experts;
    pl->k = p->top_k;
    pl->eb = p->expert_begin;
    pl->el = p->num_local;
    pl->rows_cap = p->tokens * (int64_t)(p->top_k < p->num_local ? p->top_k : p->num_local);
    pl->nslot = p->tokens * (int64_t)p->top_k;
    pl->nchunk = (int)((p->tokens + kRouteChunk - 1) / kRouteChunk);
    pl->bm = bm;
    pl->bn = bn;
    pl->n_tiles = p->d_ffn / bn;
    // wgrad K chunk: four times the mean rows per expert of the whole layer,
    // rounded up to 256, clamped to [512, kMaxChunkRows]; a pure function of
    // shapes.  Only experts holding more rows than that (skewed routing) are
    // split.  An expert holds at most `tokens` rows, so with kc >= tokens no
    // expert can split and the ordered reduction is not needed at all.
    // Splitting only pays when the layer has few weight-gradient tiles (one
    // per expert and 256x256 block of dW): with kManyWgradTiles or more every
    // compute unit already runs many tiles, and a split would only add
    // float32 partial writes and the ordered reduction, so the largest chunk
    // is taken.
    const double mean = (double)p->tokens * p->top_k / p->num_experts;
    int64_t kc = 256 * (int64_t)((4.0 * mean + 255.0) / 256.0);
    if (kc < 512) kc = 512;
    const int64_t wtiles = (int64_t)p->num_local * (p->d_model / 256) * (p->d_ffn / 256);
    if (wtiles >= kManyWgradTiles || kc > kMaxChunkRows) kc = kMaxChunkRows;
    pl->kc = (int)kc;
    pl->may_split = kc < p->tokens;
    pl->wslots = pl->may_split ? pl->rows_cap / kc : 0;
    // sum over experts of ceil(cnt/BM) <= rows_cap/BM + El; of max(1, ceil(cnt/kc)) <= El + rows_cap/kc
    pl->mt_cap = (pl->rows_cap + bm - 1) / bm + pl->el;
    pl->wu_cap = pl->el + pl->rows_cap / kc + 1;
    pl->bm2 = bf16 ? kRowTile2 : bm;
    // fc1 dgrad tiles of 192 rows (two wave rows of 96): a 256-row list with
    // few tiles per expert leaves compute units idle and splits waves 128 /
    // <128, while with many experts of few rows the extra tiles of the
    // 192-row list only re-read weights (which then bound that GEMM); so the
    // 192-row list is used when the mean expert has at least 512 rows.
    pl->fc1_list2 = bf16 && mean >= 512.0;
    pl->mt_cap2 = (pl->rows_cap + pl->bm2 - 1) / pl->bm2 + pl->el;
    pl->list2_at = kSchedHeader + 4 * (pl->mt_cap + pl->wu_cap);
    pl->aux_at = pl->list2_at + 4 * pl->mt_cap2;
    pl->pad_at = pl->aux_at + 4 * pl->wu_cap;
    pl->sched_elems = pl->pad_at + pl->el + 1;
    // sum over experts of round_up(cnt, kMxPad) <= rows_cap + el (kMxPad - 1)
    pl->rpad_cap = (pl->rows_cap + (int64_t)pl->el * (kMxPad - 1) + kMxPad - 1) / kMxPad * kMxPad;
    pl->esize = bf16 ? 2 : 4;
  }
  return MOE_OK;
}

// Workspace layout of each call: a list of aligned regions.
struct FwdWs {
  size_t hist, cursor, arows, orows, y32, total;
};
struct DgradWs {
  size_t part, dxrows, dx32, total;
};
struct WgradWs {
  size_t sched, slots1, slots2, tickets, actp, total;
  int64_t n_tickets;  // per weight gradient
};

FwdWs fwd_layout(const Plan& pl, int combine, bool atomic) {
  FwdWs w{};
  size_t o = 0;
  w.hist = o;
  o += align_up((size_t)pl.nchunk * pl.el * 4);
  w.cursor = o;
  o += align_up((size_t)pl.el * 4);
  w.arows = o;
  o += align_up((size_t)pl.rows_cap * pl.F * pl.esize);
  w.orows = o;
  if (combine) o += align_up((size_t)pl.rows_cap * pl.D * pl.esize);
  w.y32 = o;
  if (combine && atomic) o += align_up((size_t)pl.T * pl.D * 4);
  w.total = o;
  return w;
}

DgradWs dgrad_layout(const Plan& pl, int combine, bool atomic) {
  DgradWs w{};
  size_t o = 0;
  w.part = o;
  if (!atomic) o += align_up((size_t)pl.rows_cap * pl.n_tiles * 4);
  w.dxrows = o;
  if (combine) o += align_up((size_t)pl.rows_cap * pl.D * pl.esize);
  w.dx32 = o;
  if (combine && atomic) o += align_up((size_t)pl.T * pl.D * 4);
  w.total = o;
  return w;
}

// wgrad: the float32 path's split schedule, the split-K partial slots of
// both weight gradients (deterministic mode), the arrival tickets of split
// tiles (deterministic bf16: one int per partial slot and 256x256 tile, per
// weight gradient) and act_p = p relu(h)^2 [rows_cap, F].
WgradWs wgrad_layout(const Plan& pl, bool atomic) {
  WgradWs w{};
  size_t o = 0;
  w.sched = o;
  o += align_up((size_t)2 * (pl.el + 1) * 4);
  const size_t slot_bytes = align_up((size_t)pl.wslots * pl.D * pl.F * 4);
  w.slots1 = o;
  if (!atomic) o += slot_bytes;
  w.slots2 = o;
  if (!atomic) o += slot_bytes;
  w.n_tickets = (!atomic && pl.bf16) ? pl.wslots * (int64_t)(pl.D / pl.bm) * (pl.F / pl.bn) : 0;
  w.tickets = o;
  o += align_up((size_t)2 * w.n_tickets * 4);
  w.actp = o;
  o += align_up((size_t)pl.rows_cap * pl.F * pl.esize);
  w.total = o;
  return w;
}

moe_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (need > 0 && (!ws || ((uintptr_t)ws % kAlign))) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// Records the caller's stage events around each kernel of a call.
struct Stager {
  const moe_problem* p;
  hipStream_t st;
  int i = 0;
  hipError_t err = hipSuccess;
  void mark() {
    if (p->stage_events && i < p->n_stage_events) {
      hipError_t e = hipEventRecord((hipEvent_t)p->stage_events[i], st);
      if (e != hipSuccess && err == hipSuccess) err = e;
    }
    ++i;
  }
};

int64_t rowgemm_grid(const Plan& pl, int N, bool list2 = false) {
  const int64_t mtiles = list2 ? pl.mt_cap2 : pl.mt_cap;
  return grid_for_unit_rounds(mtiles * (N / pl.bn));
}

// Compute units of the current device (cached per device ordinal; the
// value never changes, so a racing first fill writes the same number).
int device_cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}

int64_t wgrad_grid(const Plan& pl, int M, int N) {
  const int64_t units = (int64_t)(pl.el + pl.wslots) * (M / pl.bm) * (N / pl.bn);
  return grid_for_units(units);
}

#define HIP_TRY(expr)                          \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return MOE_ERR_HIP;  \
  } while (0)

}  // namespace
}  // namespace moedet

using namespace moedet;

MOE_API int moe_abi_version(void) { return MOE_ABI_VERSION; }

#ifndef MOEDET_SOURCE_HASH
#define MOEDET_SOURCE_HASH "unknown"
#endif
MOE_API const char* moe_source_hash(void) { return MOEDET_SOURCE_HASH; }

MOE_API const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer argument";
    case MOE_ERR_SHAPE: return "invalid shape, alignment or expert range";
    case MOE_ERR_DTYPE: return "unsupported dtype";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_MODE: return "invalid mode or combine flag";
    case MOE_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

MOE_API moe_status moe_rows_cap(const moe_problem* p, int64_t* rows_cap) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (!rows_cap) return MOE_ERR_NULL;
  *rows_cap = pl.rows_cap;
  return MOE_OK;
}

MOE_API moe_status moe_workspace_size(const moe_problem* p, moe_mode mode, size_t* fwd_bytes,
                                      size_t* dgrad_bytes, size_t* wgrad_bytes) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (mode != MOE_DETERMINISTIC && mode != MOE_ATOMIC) return MOE_ERR_MODE;
  const bool at = mode == MOE_ATOMIC;
  if (fwd_bytes) *fwd_bytes = fwd_layout(pl, p->combine, at).total;
  if (dgrad_bytes) *dgrad_bytes = dgrad_layout(pl, p->combine, at).total;
  if (wgrad_bytes) *wgrad_bytes = wgrad_layout(pl, at).total;
  return MOE_OK;
}

MOE_API moe_status moe_sched_elems(const moe_problem* p, int64_t* elems) {
  Plan pl;
  const moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (!elems) return MOE_ERR_NULL;
  *elems = pl.sched_elems;
  return MOE_OK;
}

MOE_API const char* moe_stage_names(const moe_problem* p, moe_mode mode, int call) {
  if (validate(p, nullptr) != MOE_OK) return nullptr;
  const bool at = mode == MOE_ATOMIC;
  const bool cb = p->combine == 1;
  switch (call) {
    case 0:
      if (!at) return cb ? "route,permute_scan,permute_scatter,fc1_fwd,fc2_fwd,combine_gather"
                         : "route,permute_scan,permute_scatter,fc1_fwd,fc2_fwd";
      return cb ? "route,permute_scan,permute_scatter_atomic,fc1_fwd,fc2_fwd,zero,combine_scatter,cast"
                : "route,permute_scan,permute_scatter_atomic,fc1_fwd,fc2_fwd";
    case 1:
      if (!at) return cb ? "fc2_dgrad_dprob_partials,fc1_dgrad_dprob_combine,dx_combine_gather"
                         : "fc2_dgrad_dprob_partials,fc1_dgrad_dprob_combine";
      return cb ? "zero,fc2_dgrad_dprob_atomic,fc1_dgrad,dx_combine_scatter,cast"
                : "zero,fc2_dgrad_dprob_atomic,fc1_dgrad";
    case 2: {
      Plan pl;
      validate(p, &pl);
      if (!pl.bf16) {
        if (at) return "wgrad_prep_act_p_zero,wgrad_fc1,wgrad_fc2";
        return pl.may_split ? "wgrad_prep_act_p,wgrad_fc1,wgrad_fc2,wgrad_reduce"
                            : "wgrad_prep_act_p,wgrad_fc1,wgrad_fc2";
      }
      if (at) return "wgrad_prep_act_p_zero,wgrad_fc1_fc2";
      return "wgrad_prep_act_p,wgrad_fc1_fc2_ordered";
    }
    case 3:
      return at ? "route,permute_scan,permute_scatter_atomic" : "route,permute_scan,permute_scatter";
  }
  return nullptr;
}

namespace {

// Top-k routing, the stable permutation and the backward work list (the
// first three kernels of moe_fwd) into `routing`, with the forward
// workspace's histogram and cursor regions.
hipError_t route_enqueue(const moe_problem* p, const Plan& pl, const float* logits, const moe_routing* routing,
                         char* wsb, const FwdWs& L, bool at, Stager& sg, hipStream_t st) {
  RouteParams R{};
  R.logits = logits;
  R.T = pl.T;
  R.E = pl.E;
  R.k = pl.k;
  R.eb = pl.eb;
  R.el = pl.el;
  R.topk_idx = routing->topk_idx;
  R.topk_prob = routing->topk_prob;
  R.hist = (int32_t*)(wsb + L.hist);
  R.counts = routing->counts;
  R.offsets = routing->offsets;
  R.cursor = (int32_t*)(wsb + L.cursor);
  R.row_src = routing->row_src;
  R.row_tok = routing->row_tok;
  R.row_prob = routing->row_prob;
  R.slot_row = routing->slot_row;
  R.sched = routing->sched;
  R.bm = pl.bm;
  R.bm2 = pl.bm2;
  R.list2_at = pl.list2_at;
  R.aux_at = pl.aux_at;
  R.pad_at = pl.pad_at;
  R.kc = pl.kc;
  R.mt_cap = pl.mt_cap;
  R.nchunk = pl.nchunk;
  R.atomic = at;
  R.seed = p->debug_shuffle_seed;
  hipError_t e;
  sg.mark();
  if ((e = launch_route(R, st)) != hipSuccess) return e;
  sg.mark();
  if ((e = launch_permute_scan(R, st)) != hipSuccess) return e;
  sg.mark();
  return launch_permute_scatter(R, st);
}

// Argument checks shared by moe_fwd and moe_route.
moe_status route_check(const moe_problem* p, Plan* pl, const float* logits, const moe_routing* routing,
                       moe_mode mode) {
  moe_status s = validate(p, pl);
  if (s != MOE_OK) return s;
  if (mode != MOE_DETERMINISTIC && mode != MOE_ATOMIC) return MOE_ERR_MODE;
  if (!routing || !routing->counts || !routing->offsets || !routing->sched) return MOE_ERR_NULL;
  if (pl->T > 0 && (!logits || !routing->topk_idx || !routing->topk_prob || !routing->slot_row)) return MOE_ERR_NULL;
  if (pl->rows_cap > 0 && (!routing->row_src || !routing->row_tok || !routing->row_prob)) return MOE_ERR_NULL;
  return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_route(const moe_problem* p, const float* logits, const moe_routing* routing, void* ws,
                             size_t ws_bytes, moe_mode mode, void* stream) {
  Plan pl;
  moe_status s = route_check(p, &pl, logits, routing, mode);
  if (s != MOE_OK) return s;
  const bool at = mode == MOE_ATOMIC;
  const FwdWs L = fwd_layout(pl, p->combine, at);
  s = check_ws(ws, ws_bytes, L.total);
  if (s != MOE_OK) return s;
  Stager sg{p, (hipStream_t)stream};
  const hipError_t e = route_enqueue(p, pl, logits, routing, (char*)ws, L, at, sg, (hipStream_t)stream);
  sg.mark();
  return e == hipSuccess && sg.err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_fwd(const moe_problem* p, const float* logits, const void* x, const void* w1,
                           const void* w2, const moe_routing* routing, void* h, void* y_or_rows,
                           void* ws, size_t ws_bytes, moe_mode mode, void* stream) {
  Plan pl;
  moe_status s = route_check(p, &pl, logits, routing, mode);
  if (s != MOE_OK) return s;
  const bool at = mode == MOE_ATOMIC;
  const bool has_tok = pl.T > 0, has_rows = pl.rows_cap > 0;
  if (!w1 || !w2) return MOE_ERR_NULL;
  if (has_tok && (!x || !y_or_rows)) return MOE_ERR_NULL;
  if (has_rows && !h) return MOE_ERR_NULL;
  const FwdWs L = fwd_layout(pl, p->combine, at);
  s = check_ws(ws, ws_bytes, L.total);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  const uint64_t seed = p->debug_shuffle_seed;
  Stager sg{p, st};
  HIP_TRY(route_enqueue(p, pl, logits, routing, wsb, L, at, sg, st));

  void* orows = p->combine ? (void*)(wsb + L.orows) : y_or_rows;
  RowGemmParams G{};
  G.counts = routing->counts;
  G.offsets = routing->offsets;
  G.groups = pl.el;
  G.ncu = device_cu_count();
  G.sched = routing->sched;
  G.list_hdr = 0;
  G.list_at = kSchedHeader;
  G.seed = seed;
  // fc1: h = x[row_tok] W1_g, W1 [D][F]
  void* arows = wsb + L.arows;
  G.N = pl.F;
  G.K = pl.D;
  G.a = x;
  G.lda = pl.D;
  G.a_bytes = (uint32_t)(pl.T * pl.D * pl.esize);
  G.a_rows = routing->row_tok;
  G.b = w1;
  G.b_gstride = (int64_t)pl.D * pl.F;
  G.ldb = pl.F;
  G.b_bytes = (uint32_t)(G.b_gstride * pl.esize);
  G.c = h;
  G.ldc = pl.F;
  G.c2 = arows;
  G.ldc2 = pl.F;
  sg.mark();
  HIP_TRY(launch_rowgemm(G, kGemmFc1Fwd, pl.bf16, rowgemm_grid(pl, pl.F), st));
  // fc2: o = a W2_g with a = relu(h)^2 from the fc1 epilogue, W2 [F][D]
  G.N = pl.D;
  G.K = pl.F;
  G.a = arows;
  G.lda = pl.F;
  G.a_bytes = 0;  // rows of the tile, addressed from its first
  G.a_rows = nullptr;
  G.b = w2;
  G.b_gstride = (int64_t)pl.F * pl.D;
  G.ldb = pl.D;
  G.b_bytes = (uint32_t)(G.b_gstride * pl.esize);
  G.c = orows;
  G.ldc = pl.D;
  G.c2 = nullptr;
  sg.mark();
  HIP_TRY(launch_rowgemm(G, kGemmFc2Fwd, pl.bf16, rowgemm_grid(pl, pl.D), st));

  if (p->combine) {
    if (!at) {
      sg.mark();
      HIP_TRY(launch_gather_combine(orows, routing->slot_row, routing->topk_prob, pl.T, pl.k, pl.D, y_or_rows,
                                    pl.bf16, seed, st));
    } else {
      float* y32 = (float*)(wsb + L.y32);
      sg.mark();
      HIP_TRY(launch_zero(y32, pl.T * pl.D, st));
      sg.mark();
      HIP_TRY(launch_scatter_add(orows, routing->offsets, pl.el, routing->row_tok, routing->row_prob, pl.rows_cap,
                                 pl.D, y32, pl.bf16, seed, st));
      sg.mark();
      HIP_TRY(launch_cast(y32, y_or_rows, pl.T * pl.D, pl.bf16, st));
    }
  }
  sg.mark();
  return sg.err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

namespace {

// Argument checks of moe_bwd_dgrad_dprob (and its no-allocation variant),
// before the workspace is known.
moe_status dgrad_check(const moe_problem* p, Plan* pl, const moe_routing* routing, const void* dy, const void* w1,
                       const void* w2, const void* h, void* dx_or_rows, float* dprob, void* dh, moe_mode mode) {
  moe_status s = validate(p, pl);
  if (s != MOE_OK) return s;
  if (mode != MOE_DETERMINISTIC && mode != MOE_ATOMIC) return MOE_ERR_MODE;
  const bool has_tok = pl->T > 0, has_rows = pl->rows_cap > 0;
  if (!routing || !w1 || !w2 || !routing->counts || !routing->offsets || !routing->sched) return MOE_ERR_NULL;
  if (has_tok && (!dy || !dx_or_rows || !dprob || !routing->slot_row || !routing->topk_prob)) return MOE_ERR_NULL;
  if (has_rows && (!h || !dh || !routing->row_src || !routing->row_tok || !routing->row_prob))
    return MOE_ERR_NULL;
  return MOE_OK;
}

// The launch sequence of moe_bwd_dgrad_dprob on a checked problem and a
// workspace of at least dgrad_layout(...).total bytes.
moe_status dgrad_enqueue(const moe_problem* p, const Plan& pl, const moe_routing* routing, const void* dy,
                         const void* w1, const void* w2, const void* h, void* dx_or_rows, float* dprob, void* dh,
                         void* ws, moe_mode mode, void* stream);

}  // namespace

MOE_API moe_status moe_bwd_dgrad_dprob(const moe_problem* p, const moe_routing* routing, const void* dy,
                                       const void* w1, const void* w2, const void* h, void* dx_or_rows,
                                       float* dprob, void* dh, void* ws, size_t ws_bytes, moe_mode mode,
                                       void* stream) {
  Plan pl;
  moe_status s = dgrad_check(p, &pl, routing, dy, w1, w2, h, dx_or_rows, dprob, dh, mode);
  if (s != MOE_OK) return s;
  s = check_ws(ws, ws_bytes, dgrad_layout(pl, p->combine, mode == MOE_ATOMIC).total);
  if (s != MOE_OK) return s;
  return dgrad_enqueue(p, pl, routing, dy, w1, w2, h, dx_or_rows, dprob, dh, ws, mode, stream);
}

// ---------------------------------------------------- no-allocation variant
// The dgrad workspace of moe_bwd_dgrad_dprob_noalloc lives in this
// file-scope device array: every GPU the library runs on holds its own copy
// of kScratchBytes until the process ends.  In host code `scratch` is only a
// stand-in for the symbol; the device address of a GPU's copy comes from
// hipGetSymbolAddress with that GPU current, and only that address is ever
// handed to kernels.
namespace {
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
// Device address of the current GPU's scratch array, looked up once per
// device (with that device current, as the call runs on it).
moe_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = ptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return MOE_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

MOE_API moe_status moe_bwd_dgrad_dprob_noalloc(const moe_problem* p, const moe_routing* routing, const void* dy,
                                               const void* w1, const void* w2, const void* h, void* dx_or_rows,
                                               float* dprob, void* dh, moe_mode mode, void* stream) {
  Plan pl;
  moe_status s = dgrad_check(p, &pl, routing, dy, w1, w2, h, dx_or_rows, dprob, dh, mode);
  if (s != MOE_OK) return s;
  if (dgrad_layout(pl, p->combine, mode == MOE_ATOMIC).total > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  s = scratch_for_current_device(&ws);
  if (s != MOE_OK) return s;
  return dgrad_enqueue(p, pl, routing, dy, w1, w2, h, dx_or_rows, dprob, dh, ws, mode, stream);
}

namespace {
moe_status dgrad_enqueue(const moe_problem* p, const Plan& pl, const moe_routing* routing, const void* dy,
                         const void* w1, const void* w2, const void* h, void* dx_or_rows, float* dprob, void* dh,
                         void* ws, moe_mode mode, void* stream) {
  const bool at = mode == MOE_ATOMIC;
  const DgradWs L = dgrad_layout(pl, p->combine, at);
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  const uint64_t seed = p->debug_shuffle_seed;
  Stager sg{p, st};
  float* part = (float*)(wsb + L.part);
  float* dx32 = (float*)(wsb + L.dx32);
  void* dxrows = p->combine ? (void*)(wsb + L.dxrows) : dx_or_rows;

  if (at) {
    sg.mark();
    HIP_TRY(launch_zero(dprob, pl.nslot, st));
    if (p->combine) HIP_TRY(launch_zero(dx32, pl.T * pl.D, st));
  }
  RowGemmParams G{};
  G.counts = routing->counts;
  G.offsets = routing->offsets;
  G.groups = pl.el;
  G.ncu = device_cu_count();
  G.sched = routing->sched;
  G.list_hdr = 0;
  G.list_at = kSchedHeader;
  G.seed = seed;
  // fc2 dgrad: G = dy[row_tok] W2_g^T; W2 [F][D] read as [N=F][K=D].
  G.N = pl.F;
  G.K = pl.D;
  G.a = dy;
  G.lda = pl.D;
  G.a_bytes = (uint32_t)(pl.T * pl.D * pl.esize);
  G.a_rows = routing->row_tok;
  G.b = w2;
  G.b_gstride = (int64_t)pl.F * pl.D;
  G.ldb = pl.D;
  G.b_bytes = (uint32_t)(G.b_gstride * pl.esize);
  G.c = dh;
  G.ldc = pl.F;
  G.h = h;
  G.ldh = pl.F;
  G.row_prob = routing->row_prob;
  G.row_src = routing->row_src;
  G.part = part;
  G.n_tiles = pl.n_tiles;
  G.dprob = dprob;
  G.atomic = at;
  sg.mark();
  HIP_TRY(launch_rowgemm(G, kGemmFc2Dgrad, pl.bf16, rowgemm_grid(pl, pl.F), st));
  // fc1 dgrad: dx_rows = dh W1_g^T; W1 [D][F] read as [N=D][K=F].
  RowGemmParams G2{};
  G2.counts = routing->counts;
  G2.offsets = routing->offsets;
  G2.groups = pl.el;
  G2.ncu = device_cu_count();
  G2.sched = routing->sched;
  G2.list_hdr = pl.fc1_list2 ? 2 : 0;
  G2.list_at = pl.fc1_list2 ? pl.list2_at : kSchedHeader;
  G2.seed = seed;
  G2.N = pl.D;
  G2.K = pl.F;
  G2.a = dh;
  G2.lda = pl.F;
  G2.a_bytes = 0;  // rows of the tile, addressed from its first
  G2.a_rows = nullptr;
  G2.b = w1;
  G2.b_gstride = (int64_t)pl.D * pl.F;
  G2.ldb = pl.F;
  G2.b_bytes = (uint32_t)(G2.b_gstride * pl.esize);
  G2.c = dxrows;
  G2.ldc = pl.D;
  const int64_t gemm_grid = rowgemm_grid(pl, pl.D, pl.fc1_list2);
  int64_t side = 0;
  if (!at) {
    // the fixed-order dprob combine rides along as side units of this launch
    side = (pl.nslot + kSideSlots - 1) / kSideSlots;
    G2.part = part;
    G2.n_tiles = pl.n_tiles;
    G2.dprob = dprob;
    G2.side_slot_row = routing->slot_row;
    G2.side_nslot = pl.nslot;
    G2.side_units = (int)side;
    G2.gemm_grid = gemm_grid;
  }
  sg.mark();
  HIP_TRY(launch_rowgemm(G2, kGemmFc1Dgrad, pl.bf16, gemm_grid + side, st));
  if (p->combine) {
    if (!at) {
      sg.mark();
      HIP_TRY(launch_gather_combine(dxrows, routing->slot_row, nullptr, pl.T, pl.k, pl.D, dx_or_rows, pl.bf16,
                                    seed, st));
    } else {
      sg.mark();
      HIP_TRY(launch_scatter_add(dxrows, routing->offsets, pl.el, routing->row_tok, nullptr, pl.rows_cap, pl.D,
                                 dx32, pl.bf16, seed, st));
      sg.mark();
      HIP_TRY(launch_cast(dx32, dx_or_rows, pl.T * pl.D, pl.bf16, st));
    }
  }
  sg.mark();
  return sg.err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
}  // namespace

MOE_API moe_status moe_bwd_wgrad(const moe_problem* p, const moe_routing* routing, const void* x,
                                 const void* dy, const void* h, const void* dh, float* dw1, float* dw2,
                                 void* ws, size_t ws_bytes, moe_mode mode, void* stream) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (mode != MOE_DETERMINISTIC && mode != MOE_ATOMIC) return MOE_ERR_MODE;
  const bool at = mode == MOE_ATOMIC;
  const bool has_tok = pl.T > 0, has_rows = pl.rows_cap > 0;
  if (!routing || !dw1 || !dw2 || !routing->counts || !routing->offsets || !routing->sched) return MOE_ERR_NULL;
  if (has_tok && (!x || !dy)) return MOE_ERR_NULL;
  if (has_rows && (!h || !dh || !routing->row_tok || !routing->row_prob)) return MOE_ERR_NULL;
  const WgradWs L = wgrad_layout(pl, at);
  s = check_ws(ws, ws_bytes, L.total);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  const uint64_t seed = p->debug_shuffle_seed;
  Stager sg{p, st};
  int32_t* sched = (int32_t*)(wsb + L.sched);
  float* slots1 = (float*)(wsb + L.slots1);
  float* slots2 = (float*)(wsb + L.slots2);
  int32_t* tickets = (int32_t*)(wsb + L.tickets);
  void* act_p = wsb + L.actp;

  WgradPrepParams Q{};
  Q.counts = routing->counts;
  Q.offsets = routing->offsets;
  Q.sched = pl.bf16 ? nullptr : sched;
  Q.groups = pl.el;
  Q.M = pl.D;
  Q.N = pl.F;
  Q.kc = pl.kc;
  Q.atomic = at && pl.may_split;
  Q.dw1 = dw1;
  Q.dw2 = dw2;
  Q.slots1 = slots1;
  Q.slots2 = slots2;
  Q.h = h;
  Q.row_prob = routing->row_prob;
  Q.act_p = act_p;
  Q.tickets = tickets;
  Q.n_tickets = 2 * L.n_tickets;

  WgradParams W1{};
  W1.counts = routing->counts;
  W1.offsets = routing->offsets;
  W1.row_tok = routing->row_tok;
  W1.units = routing->sched;
  W1.units_at = kSchedHeader + 4 * pl.mt_cap;
  W1.aux_at = pl.aux_at;
  W1.sched = sched;
  W1.groups = pl.el;
  W1.kc = pl.kc;
  W1.atomic = at;
  W1.seed = seed;
  const uint32_t tok_d_bytes = (uint32_t)(pl.T * pl.D * pl.esize);
  WgradParams W2 = W1;
  // dW1_g [D][F] = x[row_tok]^T dh
  W1.M = pl.D;
  W1.N = pl.F;
  W1.a = x;
  W1.lda = pl.D;
  W1.a_bytes = tok_d_bytes;
  W1.b = dh;
  W1.ldb = pl.F;
  W1.b_bytes = 0;  // routed rows: addressed from each chunk's first row in the kernel
  W1.dw = dw1;
  W1.slots = slots1;
  W1.tickets = tickets;
  // dW2_g [F][D] = act_p^T dy[row_tok], act_p = p relu(h)^2 from the prologue
  W2.M = pl.F;
  W2.N = pl.D;
  W2.a = act_p;
  W2.lda = pl.F;
  W2.a_bytes = 0;  // routed rows: addressed from each chunk's first row in the kernel
  W2.b = dy;
  W2.ldb = pl.D;
  W2.b_bytes = tok_d_bytes;
  W2.dw = dw2;
  W2.slots = slots2;
  W2.tickets = tickets + L.n_tickets;

  // prologue grid: one 16-byte vector of act_p per thread and iteration
  const int64_t nvec = pl.rows_cap * pl.F / (pl.bf16 ? 8 : 4);
  int64_t pgrid = (nvec + 255) / 256;
  if (pgrid > 8192) pgrid = 8192;
  if (pgrid < 1) pgrid = 1;
  sg.mark();
  HIP_TRY(launch_wgrad_prep(Q, pl.bf16, pgrid, st));
  if (pl.bf16) {
    // both weight gradients in one launch; split tiles are reduced in chunk
    // order by the chunk that finishes last (deterministic mode)
    const int64_t units = (int64_t)(pl.el + pl.wslots) * (pl.D / pl.bm) * (pl.F / pl.bn);
    sg.mark();
    HIP_TRY(launch_wgrad_pair(W1, W2, device_cu_count(), grid_for_unit_rounds(2 * units), st));
  } else {
    sg.mark();
    HIP_TRY(launch_wgrad(W1, 1, pl.bf16, wgrad_grid(pl, pl.D, pl.F), st));
    sg.mark();
    HIP_TRY(launch_wgrad(W2, 2, pl.bf16, wgrad_grid(pl, pl.F, pl.D), st));
    if (!at && pl.may_split) {
      sg.mark();
      HIP_TRY(launch_wgrad_reduce(Q, 1024, st));
    }
  }
  sg.mark();
  return sg.err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_router_bwd(const moe_problem* p, const moe_routing* routing, const float* dprob,
                                  const void* x, const void* w_router, float* dlogits, float* dw_router,
                                  void* dx_router, moe_mode mode, void* stream) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (mode != MOE_DETERMINISTIC && mode != MOE_ATOMIC) return MOE_ERR_MODE;
  // the router backward needs every expert's routed rows: full layer only
  if (p->combine != 1 || p->num_local != p->num_experts) return MOE_ERR_SHAPE;
  if (!routing || !dw_router || !routing->counts || !routing->offsets) return MOE_ERR_NULL;
  if (!w_router && pl.T > 0) return MOE_ERR_NULL;
  if (pl.T > 0 && (!dprob || !x || !dlogits || !dx_router || !routing->topk_idx || !routing->topk_prob ||
                   !routing->row_tok))
    return MOE_ERR_NULL;
  RouterParams R{};
  R.T = pl.T;
  R.k = pl.k;
  R.E = pl.E;
  R.D = pl.D;
  R.topk_idx = routing->topk_idx;
  R.topk_prob = routing->topk_prob;
  R.dprob = dprob;
  R.offsets = routing->offsets;
  R.counts = routing->counts;
  R.row_tok = routing->row_tok;
  R.x = x;
  R.wr = w_router;
  R.dlogits = dlogits;
  R.dwr = dw_router;
  R.dx = dx_router;
  // dw_router row phases: a function of the shapes only (the mean routed
  // rows per expert and d_model), so the summation order is fixed
  R.phases = ((double)pl.T * pl.k / pl.E < 512.0 && pl.D % 256 == 0) ? 8 : 64;
  R.atomic = mode == MOE_ATOMIC;
  R.seed = p->debug_shuffle_seed;
  return launch_router_bwd(R, pl.bf16, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_router_fwd(const moe_problem* p, const void* x, const void* w_router, float* logits,
                                  void* stream) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (pl.T > 0 && (!x || !w_router || !logits)) return MOE_ERR_NULL;
  return launch_router_fwd(x, w_router, pl.T, pl.E, pl.D, logits, pl.bf16, p->debug_shuffle_seed,
                           (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

MOE_API moe_status moe_sgd_step(float* master, const float* grad, int64_t n, float lr, void* runtime,
                                moe_dtype dtype, void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (n < 0 || n >= ((int64_t)1 << 40)) return MOE_ERR_SHAPE;
  if (n > 0 && (!master || !grad || !runtime)) return MOE_ERR_NULL;
  return launch_sgd(master, grad, n, lr, runtime, dtype == MOE_BF16, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

MOE_API moe_status moe_mx_quantize(const void* in, moe_dtype dtype, int64_t rows, int64_t cols, uint8_t* codes,
                                   uint8_t* scales, uint64_t debug_shuffle_seed, void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (rows < 0 || cols <= 0 || cols % 32 != 0 || rows > (((int64_t)1 << 40) / cols)) return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!in || !codes || !scales) return MOE_ERR_NULL;
  if (((uintptr_t)in & 15) || ((uintptr_t)codes & 7)) return MOE_ERR_SHAPE;
  return launch_mx_quantize(in, dtype == MOE_BF16, rows, cols, codes, scales, debug_shuffle_seed,
                            (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

MOE_API moe_status moe_nvfp4_quantize(const void* in, moe_dtype dtype, int64_t rows, int64_t cols, uint8_t* codes,
                                      uint8_t* scales, float* global_scale, uint64_t debug_shuffle_seed,
                                      void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (rows < 0 || cols <= 0 || cols % 16 != 0 || rows > (((int64_t)1 << 40) / cols)) return MOE_ERR_SHAPE;
  if (!global_scale) return MOE_ERR_NULL;
  if (rows > 0 && (!in || !codes || !scales)) return MOE_ERR_NULL;
  if (((uintptr_t)in & 15) || ((uintptr_t)codes & 3)) return MOE_ERR_SHAPE;
  return launch_nvfp4_quantize(in, dtype == MOE_BF16, rows, cols, codes, scales, global_scale, debug_shuffle_seed,
                               (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

MOE_API moe_status moe_mx_dgrad_fc1(const moe_problem* p, const moe_routing* routing, const uint8_t* dh_codes,
                                    const uint8_t* dh_scales, const uint8_t* w1_codes, const uint8_t* w1_scales,
                                    void* dx_rows, void* stream) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (!pl.bf16) return MOE_ERR_DTYPE;
  if (pl.F > kMxMaxK || pl.F % 128) return MOE_ERR_SHAPE;
  if (!routing || !routing->counts || !routing->offsets || !routing->sched) return MOE_ERR_NULL;
  if (pl.rows_cap > 0 && (!dh_codes || !dh_scales || !w1_codes || !w1_scales || !dx_rows)) return MOE_ERR_NULL;
  RowGemmParams G{};
  G.counts = routing->counts;
  G.offsets = routing->offsets;
  G.groups = pl.el;
  G.N = pl.D;
  G.K = pl.F;
  G.a = dh_codes;
  G.lda = pl.F;  // bytes per row of codes
  G.a_bytes = 0;  // rows of the tile, addressed from its first
  G.b = w1_codes;
  G.b_gstride = (int64_t)pl.D * pl.F;
  G.ldb = pl.F;
  G.b_bytes = (uint32_t)((int64_t)pl.D * pl.F);
  G.c = dx_rows;
  G.ldc = pl.D;
  G.ncu = device_cu_count();
  G.sched = routing->sched;
  G.list_hdr = pl.fc1_list2 ? 2 : 0;   // the bf16 fc1 dgrad's row-tile list
  G.list_at = pl.fc1_list2 ? pl.list2_at : kSchedHeader;
  G.a_scales = dh_scales;
  G.b_scales = w1_scales;
  G.b_sgstride = (int64_t)pl.D * (pl.F / 32);
  G.seed = p->debug_shuffle_seed;
  return launch_mx_rowgemm(G, kGemmFc1Dgrad, rowgemm_grid(pl, pl.D, pl.fc1_list2), (hipStream_t)stream) ==
                 hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

MOE_API moe_status moe_mx_dgrad_fc2(const moe_problem* p, const moe_routing* routing, const uint8_t* dy_codes,
                                    const uint8_t* dy_scales, const uint8_t* w2_codes, const uint8_t* w2_scales,
                                    const void* h, float* dprob, void* dh, void* ws, size_t ws_bytes,
                                    moe_mode mode, void* stream) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (!pl.bf16) return MOE_ERR_DTYPE;
  if (mode != MOE_DETERMINISTIC && mode != MOE_ATOMIC) return MOE_ERR_MODE;
  if (pl.D > kMxMaxK) return MOE_ERR_SHAPE;
  const bool at = mode == MOE_ATOMIC;
  if (!routing || !routing->counts || !routing->offsets || !routing->sched) return MOE_ERR_NULL;
  if (pl.T > 0 && (!dy_codes || !dy_scales || !dprob || !routing->slot_row)) return MOE_ERR_NULL;
  if (pl.rows_cap > 0 && (!w2_codes || !w2_scales || !h || !dh || !routing->row_src ||
                          !routing->row_tok || !routing->row_prob))
    return MOE_ERR_NULL;
  // the partials region of the dgrad workspace (same layout as moe_bwd_dgrad_dprob)
  const DgradWs L = dgrad_layout(pl, p->combine, at);
  s = check_ws(ws, ws_bytes, L.total);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const uint64_t seed = p->debug_shuffle_seed;
  float* part = (float*)((char*)ws + L.part);
  if (at && launch_zero(dprob, pl.nslot, st) != hipSuccess) return MOE_ERR_HIP;
  RowGemmParams G{};
  G.counts = routing->counts;
  G.offsets = routing->offsets;
  G.groups = pl.el;
  G.ncu = device_cu_count();
  G.sched = routing->sched;
  G.list_hdr = 0;
  G.list_at = kSchedHeader;
  G.seed = seed;
  // G = dequant(dy)[row_tok] dequant(W2_g)^T; W2 codes [F][D] read as [N=F][K=D]
  G.N = pl.F;
  G.K = pl.D;
  G.a = dy_codes;
  G.lda = pl.D;  // bytes per row of codes
  G.a_bytes = (uint32_t)(pl.T * pl.D);
  G.a_rows = routing->row_tok;
  G.a_scales = dy_scales;
  G.b = w2_codes;
  G.b_gstride = (int64_t)pl.F * pl.D;
  G.ldb = pl.D;
  G.b_bytes = (uint32_t)G.b_gstride;
  G.b_scales = w2_scales;
  G.b_sgstride = (int64_t)pl.F * (pl.D / 32);
  G.c = dh;
  G.ldc = pl.F;
  G.h = h;
  G.ldh = pl.F;
  G.row_prob = routing->row_prob;
  G.row_src = routing->row_src;
  G.part = part;
  G.n_tiles = pl.n_tiles;
  G.dprob = dprob;
  G.atomic = at;
  if (launch_mx_rowgemm(G, kGemmFc2Dgrad, rowgemm_grid(pl, pl.F), st) != hipSuccess) return MOE_ERR_HIP;
  if (!at && launch_dprob_combine(part, routing->slot_row, pl.nslot, pl.n_tiles, dprob, seed, st) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

MOE_API moe_status moe_mx_quantize_t(const void* in, moe_dtype dtype, int64_t groups, int64_t rows, int64_t cols,
                                     uint8_t* codes, uint8_t* scales, uint64_t debug_shuffle_seed, void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (groups < 0 || rows <= 0 || rows % 32 != 0 || cols <= 0) return MOE_ERR_SHAPE;
  if (groups > (((int64_t)1 << 40) / rows) / cols) return MOE_ERR_SHAPE;
  if (groups == 0) return MOE_OK;
  if (!in || !codes || !scales) return MOE_ERR_NULL;
  if ((uintptr_t)codes & 15) return MOE_ERR_SHAPE;
  return launch_mx_quantize_t(in, dtype == MOE_BF16, groups, rows, cols, codes, scales, debug_shuffle_seed,
                              (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

MOE_API moe_status moe_mx_fwd_fc1(const moe_problem* p, const moe_routing* routing, const uint8_t* x_codes,
                                  const uint8_t* x_scales, const uint8_t* w1t_codes, const uint8_t* w1t_scales,
                                  void* h, void* act, void* stream) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (!pl.bf16) return MOE_ERR_DTYPE;
  if (pl.D > kMxMaxK || pl.D % 128) return MOE_ERR_SHAPE;
  if (!routing || !routing->counts || !routing->offsets || !routing->sched) return MOE_ERR_NULL;
  if (pl.rows_cap > 0 && (!x_codes || !x_scales || !w1t_codes || !w1t_scales || !h || !act || !routing->row_tok))
    return MOE_ERR_NULL;
  RowGemmParams G{};
  G.counts = routing->counts;
  G.offsets = routing->offsets;
  G.groups = pl.el;
  G.ncu = device_cu_count();
  G.sched = routing->sched;
  G.list_hdr = 0;
  G.list_at = kSchedHeader;
  G.seed = p->debug_shuffle_seed;
  // h = dequant(x)[row_tok] dequant(W1_g^T)^T; W1^T codes [F][D] read as [N=F][K=D]
  G.N = pl.F;
  G.K = pl.D;
  G.a = x_codes;
  G.lda = pl.D;  // bytes per row of codes
  G.a_bytes = (uint32_t)(pl.T * pl.D);
  G.a_rows = routing->row_tok;
  G.a_scales = x_scales;
  G.b = w1t_codes;
  G.b_gstride = (int64_t)pl.F * pl.D;
  G.ldb = pl.D;
  G.b_bytes = (uint32_t)G.b_gstride;
  G.b_scales = w1t_scales;
  G.b_sgstride = (int64_t)pl.F * (pl.D / 32);
  G.c = h;
  G.ldc = pl.F;
  G.c2 = act;
  G.ldc2 = pl.F;
  return launch_mx_rowgemm(G, kGemmFc1Fwd, rowgemm_grid(pl, pl.F), (hipStream_t)stream) == hipSuccess ? MOE_OK
                                                                                                     : MOE_ERR_HIP;
}

MOE_API moe_status moe_mx_fwd_fc2(const moe_problem* p, const moe_routing* routing, const uint8_t* act_codes,
                                  const uint8_t* act_scales, const uint8_t* w2t_codes, const uint8_t* w2t_scales,
                                  void* y_or_rows, void* ws, size_t ws_bytes, moe_mode mode, void* stream) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (!pl.bf16) return MOE_ERR_DTYPE;
  if (mode != MOE_DETERMINISTIC && mode != MOE_ATOMIC) return MOE_ERR_MODE;
  if (pl.F > kMxMaxK || pl.F % 128) return MOE_ERR_SHAPE;
  const bool at = mode == MOE_ATOMIC;
  if (!routing || !routing->counts || !routing->offsets || !routing->sched) return MOE_ERR_NULL;
  if (pl.T > 0 && (!y_or_rows || !routing->slot_row || !routing->topk_prob)) return MOE_ERR_NULL;
  if (pl.rows_cap > 0 && (!act_codes || !act_scales || !w2t_codes || !w2t_scales || !routing->row_tok ||
                          !routing->row_prob))
    return MOE_ERR_NULL;
  const FwdWs L = fwd_layout(pl, p->combine, at);
  s = check_ws(ws, ws_bytes, L.total);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  const uint64_t seed = p->debug_shuffle_seed;
  void* orows = p->combine ? (void*)(wsb + L.orows) : y_or_rows;
  RowGemmParams G{};
  G.counts = routing->counts;
  G.offsets = routing->offsets;
  G.groups = pl.el;
  G.ncu = device_cu_count();
  G.sched = routing->sched;
  G.list_hdr = 0;
  G.list_at = kSchedHeader;
  G.seed = seed;
  // o = dequant(act) dequant(W2_g^T)^T; W2^T codes [D][F] read as [N=D][K=F]
  G.N = pl.D;
  G.K = pl.F;
  G.a = act_codes;
  G.lda = pl.F;
  G.a_bytes = 0;  // rows of the tile, addressed from its first
  G.a_scales = act_scales;
  G.b = w2t_codes;
  G.b_gstride = (int64_t)pl.D * pl.F;
  G.ldb = pl.F;
  G.b_bytes = (uint32_t)G.b_gstride;
  G.b_scales = w2t_scales;
  G.b_sgstride = (int64_t)pl.D * (pl.F / 32);
  G.c = orows;
  G.ldc = pl.D;
  if (launch_mx_rowgemm(G, kGemmFc2Fwd, rowgemm_grid(pl, pl.D), st) != hipSuccess) return MOE_ERR_HIP;
  if (p->combine) {
    if (!at) {
      if (launch_gather_combine(orows, routing->slot_row, routing->topk_prob, pl.T, pl.k, pl.D, y_or_rows, pl.bf16,
                                seed, st) != hipSuccess)
        return MOE_ERR_HIP;
    } else {
      float* y32 = (float*)(wsb + L.y32);
      if (launch_zero(y32, pl.T * pl.D, st) != hipSuccess ||
          launch_scatter_add(orows, routing->offsets, pl.el, routing->row_tok, routing->row_prob, pl.rows_cap, pl.D,
                             y32, pl.bf16, seed, st) != hipSuccess ||
          launch_cast(y32, y_or_rows, pl.T * pl.D, pl.bf16, st) != hipSuccess)
        return MOE_ERR_HIP;
    }
  }
  return MOE_OK;
}

MOE_API moe_status moe_mx_wgrad_rows(const moe_problem* p, int64_t* rpad_cap) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (!rpad_cap) return MOE_ERR_NULL;
  *rpad_cap = pl.rpad_cap;
  return MOE_OK;
}

// Padded rows are indexed with 32-bit integers, and the GEMM addresses an
// expert's encodings from its first slice with 32-bit offsets: an expert
// holds at most T rows, so (T rounded up to 64) x max(D, F) bytes must stay
// below 2^31.
static bool mx_wgrad_fits(const Plan& pl) {
  const int64_t rows_e = (pl.T + kMxPad - 1) / kMxPad * kMxPad;
  return pl.rpad_cap < ((int64_t)1 << 31) && rows_e * (pl.D > pl.F ? pl.D : pl.F) < ((int64_t)1 << 31);
}

MOE_API moe_status moe_mx_quantize_wgrad(const moe_problem* p, const moe_routing* routing, const void* src,
                                         moe_mxw_src kind, uint8_t* codes, uint8_t* scales, void* stream) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (!pl.bf16) return MOE_ERR_DTYPE;
  if (kind != MOE_MXW_TOKEN && kind != MOE_MXW_ROW && kind != MOE_MXW_ACT_P) return MOE_ERR_SHAPE;
  if (!mx_wgrad_fits(pl)) return MOE_ERR_SHAPE;
  if (!routing || !routing->counts || !routing->offsets || !routing->sched) return MOE_ERR_NULL;
  if (pl.rows_cap == 0) return MOE_OK;
  if (!src || !codes || !scales) return MOE_ERR_NULL;
  if (kind == MOE_MXW_TOKEN && !routing->row_tok) return MOE_ERR_NULL;
  if (kind == MOE_MXW_ACT_P && !routing->row_prob) return MOE_ERR_NULL;
  if (((uintptr_t)codes | (uintptr_t)src) & 15) return MOE_ERR_SHAPE;
  MxWgradQuantParams Q{};
  Q.src = (const uint16_t*)src;
  Q.kind = (int)kind;
  Q.cols = kind == MOE_MXW_TOKEN ? pl.D : pl.F;
  Q.rpad = pl.rpad_cap;
  Q.counts = routing->counts;
  Q.offsets = routing->offsets;
  Q.poff = routing->sched + pl.pad_at;
  Q.el = pl.el;
  Q.row_tok = routing->row_tok;
  Q.row_prob = routing->row_prob;
  Q.codes = codes;
  Q.scales = scales;
  Q.seed = p->debug_shuffle_seed;
  return launch_mx_quantize_wgrad(Q, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_mx_wgrad(const moe_problem* p, const moe_routing* routing, const uint8_t* x_codes,
                                const uint8_t* x_scales, const uint8_t* dh_codes, const uint8_t* dh_scales,
                                const uint8_t* act_codes, const uint8_t* act_scales, const uint8_t* dy_codes,
                                const uint8_t* dy_scales, float* dw1, float* dw2, void* stream) {
  Plan pl;
  moe_status s = validate(p, &pl);
  if (s != MOE_OK) return s;
  if (!pl.bf16) return MOE_ERR_DTYPE;
  if (!mx_wgrad_fits(pl)) return MOE_ERR_SHAPE;
  if (!routing || !routing->sched || !dw1 || !dw2) return MOE_ERR_NULL;
  const uint8_t* ops[8] = {x_codes, x_scales, dh_codes, dh_scales, act_codes, act_scales, dy_codes, dy_scales};
  if (pl.rows_cap > 0) {
    for (int i = 0; i < 8; ++i) {
      if (!ops[i]) return MOE_ERR_NULL;
      if ((uintptr_t)ops[i] & 15) return MOE_ERR_SHAPE;
    }
  }
  MxWgradParams W{};
  W.poff = routing->sched + pl.pad_at;
  W.groups = pl.el;
  W.D = pl.D;
  W.F = pl.F;
  W.rpad = pl.rpad_cap;
  W.x_codes = x_codes;
  W.x_scales = x_scales;
  W.dh_codes = dh_codes;
  W.dh_scales = dh_scales;
  W.act_codes = act_codes;
  W.act_scales = act_scales;
  W.dy_codes = dy_codes;
  W.dy_scales = dy_scales;
  W.dw1 = dw1;
  W.dw2 = dw2;
  W.seed = p->debug_shuffle_seed;
  return launch_mx_wgrad(W, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_fingerprint(const void* data, moe_dtype dtype, int ndim, const int64_t* shape,
                                   int64_t chunk_elems, uint64_t* chunk_hashes, uint64_t* total,
                                   void* stream) {
  int width;
  switch (dtype) {
    case MOE_U8: width = 1; break;
    case MOE_BF16: width = 2; break;
    case MOE_F32:
    case MOE_I32: width = 4; break;
    case MOE_I64:
    case MOE_F64: width = 8; break;
    default: return MOE_ERR_DTYPE;
  }
  if (ndim < 0 || ndim > 8 || chunk_elems <= 0) return MOE_ERR_SHAPE;
  if (ndim > 0 && !shape) return MOE_ERR_NULL;
  if (!total) return MOE_ERR_NULL;
  int64_t n = 1;
  for (int i = 0; i < ndim; ++i) {
    if (shape[i] < 0) return MOE_ERR_SHAPE;
    if (shape[i] > 0 && n > ((int64_t)1 << 62) / shape[i]) return MOE_ERR_SHAPE;
    n *= shape[i];
  }
  const int64_t m = (n + chunk_elems - 1) / chunk_elems;
  if (m >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if (n > 0 && (!data || !chunk_hashes)) return MOE_ERR_NULL;
  uint64_t words[12];
  int nw = 0;
  words[nw++] = (uint64_t)dtype;
  words[nw++] = (uint64_t)ndim;
  for (int i = 0; i < ndim; ++i) words[nw++] = (uint64_t)shape[i];
  words[nw++] = (uint64_t)n;
  words[nw++] = (uint64_t)chunk_elems;
  hipError_t e = launch_fingerprint(data, width, n, chunk_elems, words, nw, chunk_hashes, total,
                                    (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_API moe_status moe_mfma_rate(int64_t blocks, int64_t iters, float value, float* sink, void* stream) {
  if (blocks < 1 || blocks >= ((int64_t)1 << 31) || iters < 1) return MOE_ERR_SHAPE;
  if (!sink) return MOE_ERR_NULL;
  uint32_t bits;
  memcpy(&bits, &value, 4);
  if (bits & 0xffffu) return MOE_ERR_SHAPE;  // not a bf16 value
  return launch_mfma_rate(blocks, iters, value, sink, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
