// moe_api.hip -- the C ABI (include/moe.h): argument checks, workspace layout
// and kernel launches on the caller's stream.  Every check runs before the first
// enqueue, so an error return means nothing was enqueued.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>
#include <string>

#include <algorithm>

#include "moe_internal.h"

using namespace moe;

namespace {

thread_local std::string g_last_error;
constexpr int kStageEvents = 7;
thread_local hipEvent_t g_stage_ev[kStageEvents] = {};
thread_local bool g_stage_on = false;

void stage(int i, hipStream_t s) {
  if (g_stage_on && g_stage_ev[i]) (void)hipEventRecord(g_stage_ev[i], s);
}

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr unsigned kKnownFlags =
    MOE_F_LOGITS_GIVEN | MOE_F_VALIDATE_ONLY | MOE_F_NONDETERMINISTIC_COMBINE | MOE_F_BF16_ROWS;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define REQUIRE(cond, ...)                                       \
  do {                                                           \
    if (!(cond)) return fail(MOE_ERR_INVALID_ARG, __VA_ARGS__);  \
  } while (0)

#define REQUIRE_PTR(p, name)                                                       \
  do {                                                                             \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s must not be NULL", name);       \
    if (!aligned((p), 16)) return fail(MOE_ERR_INVALID_ARG, "%s must be 16-byte aligned", name); \
  } while (0)

#define OPT_PTR(p, name)                                                            \
  do {                                                                              \
    if ((p) && !aligned((p), 16))                                                   \
      return fail(MOE_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);         \
  } while (0)

moe_status check_common(int T, int E, int k, unsigned flags) {
  REQUIRE((flags & ~kKnownFlags) == 0, "unknown flag bits 0x%x", flags & ~kKnownFlags);
  REQUIRE(T >= 0, "T must be >= 0 (got %d)", T);
  REQUIRE(E >= 1, "n_experts must be >= 1 (got %d)", E);
  REQUIRE(k >= 1 && k <= E, "top_k must be in [1, n_experts] (got k=%d, E=%d)", k, E);
  if (E > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d unsupported", kMaxExperts);
  if (k > kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "top_k > %d unsupported", kMaxTopK);
  REQUIRE((long long)T * k < (1ll << 30), "T*k too large");
  return MOE_OK;
}

bool valid_dtype(moe_dtype d) { return d == MOE_DT_F32 || d == MOE_DT_BF16; }

moe_status check_experts(const moe_experts* w, moe_dtype xdt, int d, int F, moe_act act,
                         const char* what) {
  REQUIRE(w, "%s experts must not be NULL", what);
  REQUIRE(act == MOE_ACT_SWIGLU || act == MOE_ACT_RELU, "unknown activation %d", (int)act);
  REQUIRE(d >= 8 && d % 8 == 0, "d_model must be a positive multiple of 8 (got %d)", d);
  REQUIRE(F >= 8 && F % 8 == 0, "%s d_ff must be a positive multiple of 8 (got %d)", what, F);
  if (w->q_up) {
    if (xdt != MOE_DT_BF16)
      return fail(MOE_ERR_UNSUPPORTED, "%s INT4 experts need bf16 activations", what);
    REQUIRE(d % 128 == 0 && F % 128 == 0,
            "%s INT4 experts need d_model and d_ff multiples of 128 (got %d, %d)", what, d, F);
    REQUIRE(w->q_down, "%s INT4 q_down must not be NULL", what);
    if (act == MOE_ACT_SWIGLU) REQUIRE(w->q_gate, "%s INT4 q_gate must not be NULL", what);
    const moe_w4* qs[3] = {w->q_gate, w->q_up, w->q_down};
    for (int i = 0; i < 3; ++i) {
      if (!qs[i]) continue;
      REQUIRE_PTR(qs[i]->q, "INT4 q");
      REQUIRE(qs[i]->scale && qs[i]->zero, "INT4 scale/zero must not be NULL");
      REQUIRE(aligned(qs[i]->scale, 2) && aligned(qs[i]->zero, 2), "INT4 scale/zero misaligned");
    }
    return MOE_OK;
  }
  REQUIRE(w->dtype == xdt, "%s weight dtype (%d) must equal the activation dtype (%d)", what,
          (int)w->dtype, (int)xdt);
  REQUIRE_PTR(w->w_up, "w_up");
  REQUIRE_PTR(w->w_down, "w_down");
  if (act == MOE_ACT_SWIGLU) REQUIRE_PTR(w->w_gate, "w_gate");
  return MOE_OK;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  }
};

struct LayerWs {
  float* logits;
  int32_t *idx, *counts, *offsets, *row_assign, *assign_row;
  float* gates;
  double* lis;
  void* perm_ws;
  void* H;
  float* y_rows;           // down_splits partial copies of [T*k][d]
  int down_splits;
  void* Hs;
  // replica layer: the split routing over E+1 slots
  int32_t *counts2, *offsets2, *row_assign2, *assign_row2;
  double* lis2;
  float* y_shared;
  // replica layer with many rows: the replica's projections decoded to bf16
  void *rep_gate, *rep_up, *rep_down;
  size_t total;
};

// scratch of the routing step: the permutation's block counts, or for the
// one-workgroup path the router GEMM's block partials (never both)
size_t route_ws_bytes(const moe_layer_desc* L, int T) {
  const int E = L->n_experts, k = L->top_k;
  return std::max(permute_ws_bytes(T, E, k), route_part_bytes(L->act_dtype, T, L->d_model, E, k));
}

// A replica slot with many rows (the tiled path) runs the bf16 tile kernels on
// its projections decoded once per call into the workspace (the INT4 tile
// kernel stages weights through registers and is several times slower; the
// decoded copy is a few MB per projection); decode sizes stream the INT4
// weights directly.
bool replica_decoded(int T) { return T > 64; }

LayerWs carve_layer(const moe_layer_desc* L, int T, void* ws, bool replica = false) {
  const int E = L->n_experts, k = L->top_k, d = L->d_model, F = L->d_ff;
  const size_t n = (size_t)T * k;
  const size_t esz = L->act_dtype == MOE_DT_F32 ? 4 : 2;
  Carver c(ws);
  LayerWs w;
  w.logits = (float*)c.take((size_t)T * E * 4);
  w.idx = (int32_t*)c.take(n * 4);
  w.gates = (float*)c.take(n * 4);
  w.counts = (int32_t*)c.take((size_t)E * 4);
  w.offsets = (int32_t*)c.take((size_t)(E + 1) * 4);
  w.row_assign = (int32_t*)c.take(n * 4);
  w.assign_row = (int32_t*)c.take(n * 4);
  w.lis = (double*)c.take(8);
  w.perm_ws = c.take(route_ws_bytes(L, T));
  w.H = c.take(n * F * esz);
  // a replica layer at decode sizes runs its slot E through a separate INT4
  // pass that writes whole rows: no K slices there
  w.down_splits = (replica && !replica_decoded(T))
                      ? 1
                      : ffn_down_splits(T, d, F, E, k, L->act_dtype, &L->routed);
  w.y_rows = (float*)c.take(n * d * 4 * w.down_splits);
  const int Fs = L->n_shared * L->d_ff_shared;
  w.Hs = L->n_shared ? c.take((size_t)T * Fs * esz) : nullptr;
  w.y_shared = L->n_shared ? (float*)c.take((size_t)T * d * 4) : nullptr;
  w.counts2 = w.offsets2 = w.row_assign2 = w.assign_row2 = nullptr;
  w.lis2 = nullptr;
  w.rep_gate = w.rep_up = w.rep_down = nullptr;
  if (replica && replica_decoded(T)) {
    if (L->act == MOE_ACT_SWIGLU) w.rep_gate = c.take((size_t)F * d * 2);
    w.rep_up = c.take((size_t)F * d * 2);
    w.rep_down = c.take((size_t)d * F * 2);
  }
  if (replica) {
    w.counts2 = (int32_t*)c.take((size_t)(E + 1) * 4);
    w.offsets2 = (int32_t*)c.take((size_t)(E + 2) * 4);
    w.row_assign2 = (int32_t*)c.take(n * 4);
    w.assign_row2 = (int32_t*)c.take(n * 4);
    w.lis2 = (double*)c.take(8);
  }
  w.total = c.off;
  return w;
}

// routed = false: the routed experts come from elsewhere (nested weights)
moe_status check_layer(const moe_layer_desc* L, int T, unsigned flags, bool routed = true) {
  REQUIRE(L, "layer descriptor must not be NULL");
  moe_status s = check_common(T, L->n_experts, L->top_k, flags);
  if (s != MOE_OK) return s;
  REQUIRE(valid_dtype(L->act_dtype), "unknown activation dtype %d", (int)L->act_dtype);
  if (routed) {
    s = check_experts(&L->routed, L->act_dtype, L->d_model, L->d_ff, L->act, "routed");
    if (s != MOE_OK) return s;
  }
  if (!(flags & MOE_F_LOGITS_GIVEN)) REQUIRE_PTR(L->w_router, "w_router");
  OPT_PTR(L->b_router, "b_router");
  REQUIRE(L->n_shared >= 0, "n_shared must be >= 0");
  if (L->n_shared > 0) {
    REQUIRE(L->d_ff_shared >= 8 && L->d_ff_shared % 8 == 0,
            "d_ff_shared must be a positive multiple of 8");
    s = check_experts(&L->shared, L->act_dtype, L->d_model, L->n_shared * L->d_ff_shared,
                      MOE_ACT_SWIGLU, "shared");
    if (s != MOE_OK) return s;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_set_stage_events(void* const* events, int n) {
  if (!events) {
    g_stage_on = false;
    return ok();
  }
  REQUIRE(n == kStageEvents, "moe_set_stage_events needs %d events (got %d)", kStageEvents, n);
  for (int i = 0; i < kStageEvents; ++i) g_stage_ev[i] = (hipEvent_t)events[i];
  g_stage_on = true;
  return ok();
}

moe_status moe_route_topk(const void* x, moe_dtype xdt, const void* w_router,
                          const float* b_router, int T, int d, int E, int k, float* logits,
                          int32_t* topk_idx, float* topk_gate, unsigned flags, void* stream) {
  moe_status s = check_common(T, E, k, flags);
  if (s != MOE_OK) return s;
  REQUIRE(valid_dtype(xdt), "unknown dtype %d", (int)xdt);
  REQUIRE(d >= 8 && d % 8 == 0, "d must be a positive multiple of 8 (got %d)", d);
  const bool given = flags & MOE_F_LOGITS_GIVEN;
  if (!given) {
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(w_router, "w_router");
  }
  OPT_PTR(b_router, "b_router");
  REQUIRE_PTR(logits, "logits");
  REQUIRE_PTR(topk_idx, "topk_idx");
  OPT_PTR(topk_gate, "topk_gate");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  if (T == 0) return ok();
  return hip_status(launch_route_topk(x, xdt, w_router, b_router, T, d, E, k, logits, topk_idx,
                                      topk_gate, given, (hipStream_t)stream),
                    "moe_route_topk launch");
}

size_t moe_permute_workspace_size(int T, int E, int k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  return permute_ws_bytes(T, E, k);
}

moe_status moe_permute(const int32_t* topk_idx, int T, int E, int k, int32_t* counts,
                       int32_t* offsets, int32_t* row_assign, int32_t* assign_row, double* lis,
                       void* ws, size_t ws_bytes, unsigned flags, void* stream) {
  moe_status s = check_common(T, E, k, flags);
  if (s != MOE_OK) return s;
  if (T > 0) REQUIRE_PTR(topk_idx, "topk_idx");
  REQUIRE_PTR(counts, "counts");
  REQUIRE_PTR(offsets, "offsets");
  OPT_PTR(row_assign, "row_assign");
  OPT_PTR(assign_row, "assign_row");
  OPT_PTR(lis, "lis");
  const size_t need = permute_ws_bytes(T, E, k);
  if (need && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "moe_permute needs %zu workspace bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  OPT_PTR(ws, "ws");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  return hip_status(launch_permute(topk_idx, T, E, k, counts, offsets, row_assign, assign_row,
                                   lis, ws, (hipStream_t)stream),
                    "moe_permute launch");
}

size_t moe_grouped_ffn_workspace_size(int T, int d, int F, int E, int k, moe_act act,
                                      const moe_experts* w) {
  (void)d; (void)E; (void)act;
  if (T < 0 || F < 0 || k < 1 || !w) return 0;
  const moe_dtype dt = w->q_up ? MOE_DT_BF16 : w->dtype;
  return ffn_ws_bytes(T * k, F, dt);
}

moe_status moe_grouped_ffn(const void* x, moe_dtype xdt, int T, int d, int F, int E, int k,
                           moe_act act, const moe_experts* w, const int32_t* offsets,
                           const int32_t* row_assign, const float* topk_gate, float* y_rows,
                           void* ws, size_t ws_bytes, unsigned flags, void* stream) {
  moe_status s = check_common(T, E, k, flags);
  if (s != MOE_OK) return s;
  REQUIRE(valid_dtype(xdt), "unknown dtype %d", (int)xdt);
  s = check_experts(w, xdt, d, F, act, "routed");
  if (s != MOE_OK) return s;
  if (!offsets) REQUIRE(E == 1 && k == 1, "offsets == NULL requires E == 1 and k == 1");
  if (!row_assign) REQUIRE(k == 1, "row_assign == NULL requires k == 1");
  if (T > 0) REQUIRE_PTR(x, "x");
  REQUIRE_PTR(y_rows, "y_rows");
  OPT_PTR(offsets, "offsets");
  OPT_PTR(row_assign, "row_assign");
  OPT_PTR(topk_gate, "topk_gate");
  const size_t need = moe_grouped_ffn_workspace_size(T, d, F, E, k, act, w);
  if (need && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "moe_grouped_ffn needs %zu workspace bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  OPT_PTR(ws, "ws");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  if (T == 0) return ok();
  FfnProblem p{};
  p.T = T; p.d = d; p.F = F; p.E = E; p.k = k; p.act = act;
  p.dt = w->q_up ? MOE_DT_BF16 : xdt;
  p.x = x; p.w = w; p.offsets = offsets; p.row_assign = row_assign; p.gate = topk_gate;
  p.y_rows = y_rows; p.H = ws; p.rows = T * k;
  return hip_status(launch_grouped_ffn(p, (hipStream_t)stream), "moe_grouped_ffn launch");
}

moe_status moe_combine(const float* y_rows, const int32_t* assign_row, int T, int k, int d,
                       const float* y_shared, void* y, moe_dtype ydt, unsigned flags,
                       void* stream) {
  REQUIRE((flags & ~kKnownFlags) == 0, "unknown flag bits");
  REQUIRE(T >= 0, "T must be >= 0");
  REQUIRE(k >= 1 && k <= kMaxTopK, "top_k must be in [1, %d]", kMaxTopK);
  REQUIRE(d >= 8 && d % 8 == 0, "d must be a positive multiple of 8 (got %d)", d);
  REQUIRE(valid_dtype(ydt), "unknown output dtype %d", (int)ydt);
  if (T > 0) {
    REQUIRE_PTR(y_rows, "y_rows");
    REQUIRE_PTR(assign_row, "assign_row");
    REQUIRE_PTR(y, "y");
  }
  OPT_PTR(y_shared, "y_shared");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  return hip_status(launch_combine(y_rows, assign_row, T, k, d, y_shared, y, ydt,
                                   (hipStream_t)stream),
                    "moe_combine launch");
}

moe_status moe_workspace_size(const moe_layer_desc* L, int T, size_t* bytes) {
  REQUIRE(bytes, "bytes must not be NULL");
  moe_status s = check_layer(L, T, 0);
  if (s != MOE_OK) return s;
  *bytes = carve_layer(L, T, nullptr).total;
  return ok();
}

}  // extern "C"

namespace {

moe_status check_replica(const moe_layer_desc* L, const moe_replica* R) {
  REQUIRE(R, "replica must not be NULL");
  REQUIRE(R->expert >= 0 && R->expert < L->n_experts, "replica expert %d out of [0, %d)",
          R->expert, L->n_experts);
  if (L->act_dtype != MOE_DT_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the INT4 replica needs bf16 activations");
  moe_experts q{};
  q.dtype = MOE_DT_BF16;
  q.q_gate = R->q_gate;
  q.q_up = R->q_up;
  q.q_down = R->q_down;
  REQUIRE(R->q_up, "replica q_up must not be NULL");
  return check_experts(&q, MOE_DT_BF16, L->d_model, L->d_ff, L->act, "replica");
}

// Routing and the permutation of a layer call (one workgroup for decode
// sizes, else the route and permute kernels); stage event 1 between them.
hipError_t route_and_permute(const moe_layer_desc* L, const void* x, int T, float* logits,
                             int32_t* idx, float* gates, int32_t* counts, int32_t* offsets,
                             int32_t* row_assign, int32_t* assign_row, double* lis, void* perm_ws,
                             unsigned flags, hipStream_t st) {
  const int E = L->n_experts, k = L->top_k, d = L->d_model;
  const bool given = (flags & MOE_F_LOGITS_GIVEN) != 0;
  if (route_permute_small_applies(L->act_dtype, T, E, k)) {
    hipError_t e = launch_route_permute_small(x, L->w_router, L->b_router, T, d, E, k, logits, idx,
                                              gates, given, counts, offsets, row_assign,
                                              assign_row, lis, (float*)perm_ws, st);
    stage(1, st);
    return e;
  }
  hipError_t e = launch_route_topk(x, L->act_dtype, L->w_router, L->b_router, T, d, E, k, logits,
                                   idx, gates, given, st);
  if (e != hipSuccess) return e;
  stage(1, st);
  return launch_permute(idx, T, E, k, counts, offsets, row_assign, assign_row, lis, perm_ws, st);
}

// The layer; with R, expert R->expert's odd-ranked assignments run on the
// replica as slot E.
moe_status layer_forward_impl(const moe_layer_desc* L, const moe_replica* R, const void* x, int T,
                              void* y, moe_dtype ydt, moe_aux* aux, double* lis_base, void* ws,
                              size_t ws_bytes, unsigned flags, void* stream) {
  moe_status s = check_layer(L, T, flags);
  if (s != MOE_OK) return s;
  if (R) {
    s = check_replica(L, R);
    if (s != MOE_OK) return s;
    OPT_PTR(lis_base, "lis_base");
  }
  REQUIRE(valid_dtype(ydt), "unknown output dtype %d", (int)ydt);
  if (T > 0) {
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(y, "y");
  }
  if (aux) {
    OPT_PTR(aux->logits, "aux.logits"); OPT_PTR(aux->idx, "aux.idx");
    OPT_PTR(aux->gates, "aux.gates"); OPT_PTR(aux->counts, "aux.counts");
    OPT_PTR(aux->offsets, "aux.offsets"); OPT_PTR(aux->row_assign, "aux.row_assign");
    OPT_PTR(aux->assign_row, "aux.assign_row"); OPT_PTR(aux->lis, "aux.lis");
  }
  if ((flags & MOE_F_LOGITS_GIVEN) && !(aux && aux->logits))
    return fail(MOE_ERR_INVALID_ARG, "MOE_F_LOGITS_GIVEN needs aux->logits");
  const size_t need = carve_layer(L, T, nullptr, R != nullptr).total;
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "the layer needs %zu workspace bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  REQUIRE(aligned(ws, 256), "ws must be 256-byte aligned");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  if (T == 0) return ok();

  hipStream_t st = (hipStream_t)stream;
  LayerWs w = carve_layer(L, T, ws, R != nullptr);
  const int E = L->n_experts, k = L->top_k, d = L->d_model;
  float* logits = (aux && aux->logits) ? aux->logits : w.logits;
  int32_t* idx = (aux && aux->idx) ? aux->idx : w.idx;
  float* gates = (aux && aux->gates) ? aux->gates : w.gates;
  // the router's own routing (E slots); with a replica, aux receives the split
  int32_t* counts = (!R && aux && aux->counts) ? aux->counts : w.counts;
  int32_t* offsets = (!R && aux && aux->offsets) ? aux->offsets : w.offsets;
  int32_t* row_assign = (!R && aux && aux->row_assign) ? aux->row_assign : w.row_assign;
  int32_t* assign_row = (!R && aux && aux->assign_row) ? aux->assign_row : w.assign_row;
  double* lis = R ? (lis_base ? lis_base : w.lis) : ((aux && aux->lis) ? aux->lis : w.lis);

  FfnProblem p{};
  p.T = T; p.d = d; p.F = L->d_ff; p.E = E; p.k = k; p.act = L->act;
  p.dt = L->act_dtype; p.x = x; p.w = &L->routed;
  p.gate = gates; p.y_rows = w.y_rows; p.H = w.H; p.rows = T * k;
  p.down_splits = w.down_splits;
  // decode sizes: route, top-k and permutation in one workgroup.  When every
  // output element receives at most two gate-scaled rows (weight streaming
  // with k <= 2, no shared experts), the down pass adds them straight into y,
  // zeroed by the gate/up grid: fp32 addition of two terms onto zero gives
  // the same value in either order, so y stays run-to-run deterministic and
  // the combine launch goes away
  const bool small = !R && route_permute_small_applies(L->act_dtype, T, E, k);
  const bool direct = !R && ydt == MOE_DT_F32 && L->n_shared == 0 && ffn_direct_applies(p);
  p.zero_y = direct ? (float*)y : nullptr;
  stage(0, st);
  hipError_t e;
  if (small) {
    e = launch_route_permute_small(x, L->w_router, L->b_router, T, d, E, k, logits, idx, gates,
                                   (flags & MOE_F_LOGITS_GIVEN) != 0, counts, offsets, row_assign,
                                   assign_row, lis, (float*)w.perm_ws, st);
    if (e != hipSuccess) return hip_status(e, "route and permute");
    stage(1, st);
  } else {
    e = launch_route_topk(x, L->act_dtype, L->w_router, L->b_router, T, d, E, k, logits, idx,
                          gates, (flags & MOE_F_LOGITS_GIVEN) != 0, st);
    if (e != hipSuccess) return hip_status(e, "route_topk");
    stage(1, st);
    e = launch_permute(idx, T, E, k, counts, offsets, row_assign, assign_row, lis, w.perm_ws, st);
    if (e != hipSuccess) return hip_status(e, "permute");
  }
  // rows of expert-major order used by the FFN and the combine
  const int32_t* f_offsets = offsets;
  const int32_t* f_row_assign = row_assign;
  const int32_t* f_assign_row = assign_row;
  if (R) {
    int32_t* c2 = (aux && aux->counts) ? aux->counts : w.counts2;
    int32_t* o2 = (aux && aux->offsets) ? aux->offsets : w.offsets2;
    int32_t* ra2 = (aux && aux->row_assign) ? aux->row_assign : w.row_assign2;
    int32_t* ar2 = (aux && aux->assign_row) ? aux->assign_row : w.assign_row2;
    double* l2 = (aux && aux->lis) ? aux->lis : w.lis2;
    e = launch_replica_remap(idx, counts, offsets, assign_row, T, E, k, R->expert, nullptr, c2, o2,
                             ra2, ar2, l2, st);
    if (e != hipSuccess) return hip_status(e, "replica split");
    f_offsets = o2;
    f_row_assign = ra2;
    f_assign_row = ar2;
  }
  stage(2, st);
  p.offsets = f_offsets;
  p.row_assign = f_row_assign;
  p.y_direct = direct ? (float*)y : nullptr;
  p.rows_bf16 = (flags & MOE_F_BF16_ROWS) != 0 && !direct && ffn_rows_bf16_applies(p);
  // the replica (slot E): with many rows its INT4 projections are decoded to
  // bf16 and it runs as one more expert of the same tiled launches, so its
  // tiles share the chip with the others'; at decode sizes (or shapes off the
  // 256x256 path) it runs as a second pass over its rows with the INT4 weights
  moe_experts q{};
  q.dtype = MOE_DT_BF16;
  bool rep_joined = false;
  if (R && w.rep_up) {
    const int F = L->d_ff;
    if (w.rep_gate) {
      e = launch_dequant_int4(R->q_gate, F, d, w.rep_gate, st);
      if (e != hipSuccess) return hip_status(e, "replica decode");
    }
    e = launch_dequant_int4(R->q_up, F, d, w.rep_up, st);
    if (e == hipSuccess) e = launch_dequant_int4(R->q_down, d, F, w.rep_down, st);
    if (e != hipSuccess) return hip_status(e, "replica decode");
    q.w_gate = w.rep_gate;
    q.w_up = w.rep_up;
    q.w_down = w.rep_down;
    // (the 256x256 tile map scans up to 128 experts' row counts)
    rep_joined = d % 128 == 0 && F % 128 == 0 && E + 1 <= 128;
  } else if (R) {
    q.q_gate = R->q_gate;
    q.q_up = R->q_up;
    q.q_down = R->q_down;
  }
  if (rep_joined) {
    p.E = E + 1;
    p.xw = &q;
    p.xslot = E;
  }
  e = launch_grouped_ffn(p, st, g_stage_on ? g_stage_ev[3] : nullptr);
  if (e != hipSuccess) return hip_status(e, "grouped_ffn");
  if (R && !rep_joined) {
    // slot E: one expert whose rows start at offsets[E] (absolute rows, so the
    // same H and y_rows buffers and K slices)
    FfnProblem r = p;
    r.E = 1;
    r.w = &q;
    r.offsets = f_offsets + E;
    e = launch_grouped_ffn(r, st);
    if (e != hipSuccess) return hip_status(e, "replica ffn");
  }
  stage(4, st);
  if (L->n_shared > 0) {
    FfnProblem q{};
    q.T = T; q.d = d; q.F = L->n_shared * L->d_ff_shared; q.E = 1; q.k = 1;
    q.act = MOE_ACT_SWIGLU; q.dt = L->act_dtype; q.x = x; q.w = &L->shared;
    q.offsets = nullptr; q.row_assign = nullptr; q.gate = nullptr;
    q.y_rows = w.y_shared; q.H = w.Hs; q.rows = T;
    e = launch_grouped_ffn(q, st);
    if (e != hipSuccess) return hip_status(e, "shared experts");
  }
  stage(5, st);
  if (!direct)
    e = launch_combine(w.y_rows, f_assign_row, T, k, d, w.y_shared, y, ydt, st, w.down_splits,
                       (size_t)T * k * d, p.rows_bf16);
  stage(6, st);
  return hip_status(e, "combine");
}

}  // namespace

extern "C" {

moe_status moe_layer_forward(const moe_layer_desc* L, const void* x, int T, void* y,
                             moe_dtype ydt, moe_aux* aux, void* ws, size_t ws_bytes,
                             unsigned flags, void* stream) {
  return layer_forward_impl(L, nullptr, x, T, y, ydt, aux, nullptr, ws, ws_bytes, flags, stream);
}

}  // extern "C"

// ---- the layer without a caller workspace -----------------------------------
// The workspace of moe_layer_forward lives in one file-scope device array.
// Each device holds its own copy; host code never passes the array's name to a
// kernel (on the host it is only a stand-in), it passes the address that
// hipGetSymbolAddress returned for the current device.

namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kScratchDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_addr[kScratchDevices];

// Device address of this device's scratch array, looked up once per device.
moe_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: scratch addresses are kept for devices 0..%d",
                dev, kScratchDevices - 1);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
      if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

moe_status moe_layer_forward_noalloc(const moe_layer_desc* L, const void* x, int T, void* y,
                                     moe_dtype ydt, moe_aux* aux, unsigned flags, void* stream) {
  moe_status s = check_layer(L, T, flags);
  if (s != MOE_OK) return s;
  const size_t need = carve_layer(L, T, nullptr).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_layer_forward_noalloc: T = %d needs %zu bytes of scratch, above the "
                "static %zu bytes; call moe_layer_forward with a workspace instead",
                T, need, kScratchBytes);
  // no device is touched for a validation-only or empty call: any 256-byte
  // aligned address stands in for the scratch (it is never dereferenced)
  void* ws = (void*)(uintptr_t)256;
  if (!(flags & MOE_F_VALIDATE_ONLY) && T > 0) {
    s = scratch_address(&ws);
    if (s != MOE_OK) return s;
  }
  return layer_forward_impl(L, nullptr, x, T, y, ydt, aux, nullptr, ws, kScratchBytes, flags,
                            stream);
}

moe_status moe_layer_forward_replica(const moe_layer_desc* L, const moe_replica* R,
                                     const void* x, int T, void* y, moe_dtype ydt, moe_aux* aux,
                                     double* lis_base, void* ws, size_t ws_bytes, unsigned flags,
                                     void* stream) {
  REQUIRE(R, "replica must not be NULL");
  return layer_forward_impl(L, R, x, T, y, ydt, aux, lis_base, ws, ws_bytes, flags, stream);
}

moe_status moe_replica_workspace_size(const moe_layer_desc* L, int T, size_t* bytes) {
  REQUIRE(bytes, "bytes must not be NULL");
  moe_status s = check_layer(L, T, 0);
  if (s != MOE_OK) return s;
  *bytes = carve_layer(L, T, nullptr, true).total;
  return ok();
}

moe_status moe_replica_split(const int32_t* topk_idx, const int32_t* counts,
                             const int32_t* offsets, const int32_t* assign_row, int T, int E,
                             int k, int heavy, int32_t* idx_out, int32_t* counts_out,
                             int32_t* offsets_out, int32_t* row_assign_out,
                             int32_t* assign_row_out, double* lis_out, unsigned flags,
                             void* stream) {
  moe_status s = check_common(T, E, k, flags);
  if (s != MOE_OK) return s;
  REQUIRE(heavy >= 0 && heavy < E, "heavy expert %d out of [0, %d)", heavy, E);
  REQUIRE_PTR(counts, "counts");
  REQUIRE_PTR(offsets, "offsets");
  if (T > 0) {
    REQUIRE_PTR(topk_idx, "topk_idx");
    REQUIRE_PTR(assign_row, "assign_row");
  }
  OPT_PTR(idx_out, "idx_out"); OPT_PTR(counts_out, "counts_out");
  OPT_PTR(offsets_out, "offsets_out"); OPT_PTR(row_assign_out, "row_assign_out");
  OPT_PTR(assign_row_out, "assign_row_out"); OPT_PTR(lis_out, "lis_out");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  return hip_status(launch_replica_remap(topk_idx, counts, offsets, assign_row, T, E, k, heavy,
                                         idx_out, counts_out, offsets_out, row_assign_out,
                                         assign_row_out, lis_out, (hipStream_t)stream),
                    "moe_replica_split launch");
}

}  // extern "C"

// ---- nested (matryoshka) low-bit experts -----------------------------------

namespace {

moe_status check_mwq_experts(const moe_mwq_experts* w, int T, int d, int F, int k, moe_act act) {
  REQUIRE(w, "nested experts must not be NULL");
  REQUIRE(act == MOE_ACT_SWIGLU || act == MOE_ACT_RELU, "unknown activation %d", (int)act);
  REQUIRE(d >= 128 && d % 128 == 0 && F >= 128 && F % 128 == 0,
          "nested experts need d_model and d_ff positive multiples of 128 (got %d, %d)", d, F);
  REQUIRE(w->up && w->down, "nested experts: up and down must not be NULL");
  if (act == MOE_ACT_SWIGLU) REQUIRE(w->gate, "nested experts: gate must not be NULL for SwiGLU");
  const moe_wmwq* ms[3] = {act == MOE_ACT_SWIGLU ? w->gate : nullptr, w->up, w->down};
  for (int i = 0; i < 3; ++i) {
    const moe_wmwq* m = ms[i];
    if (!m) continue;
    REQUIRE_PTR(m->q2, "nested q2");
    REQUIRE_PTR(m->p3, "nested p3");
    REQUIRE_PTR(m->p4, "nested p4");
    REQUIRE(m->s2 && m->z2 && m->a3 && m->a4, "nested s2/z2/a3/a4 must not be NULL");
    REQUIRE(aligned(m->s2, 8) && aligned(m->z2, 8) && aligned(m->a3, 8) && aligned(m->a4, 8),
            "nested s2/z2/a3/a4 must be 8-byte aligned");
  }
  if (const char* why = mwq_ffn_unsupported(T, d, F, k)) return fail(MOE_ERR_UNSUPPORTED, "%s", why);
  return MOE_OK;
}

size_t mwq_group_ws_bytes(int T, int E, int k) {
  return align_up((size_t)T * k * 4) + align_up(permute_ws_bytes(T, 3 * E, k));
}

struct MwqLayerWs {
  LayerWs base;
  int32_t *gidx, *counts3, *offsets3, *row_assign3, *assign_row3;
  void* gperm_ws;
  size_t total;
};

MwqLayerWs carve_mwq_layer(const moe_layer_desc* L, int T, void* ws) {
  // the router's own routing, H, y_rows and the shared experts as in the plain
  // layer (one K slice), then the (expert, width) grouping
  const int E = L->n_experts, k = L->top_k, d = L->d_model, F = L->d_ff;
  const size_t n = (size_t)T * k;
  Carver c(ws);
  MwqLayerWs m;
  LayerWs& w = m.base;
  w.logits = (float*)c.take((size_t)T * E * 4);
  w.idx = (int32_t*)c.take(n * 4);
  w.gates = (float*)c.take(n * 4);
  w.counts = (int32_t*)c.take((size_t)E * 4);
  w.offsets = (int32_t*)c.take((size_t)(E + 1) * 4);
  w.row_assign = (int32_t*)c.take(n * 4);
  w.assign_row = (int32_t*)c.take(n * 4);
  w.lis = (double*)c.take(8);
  w.perm_ws = c.take(route_ws_bytes(L, T));
  w.H = c.take(n * F * 2);
  w.down_splits = 1;
  w.y_rows = (float*)c.take(n * d * 4);
  const int Fs = L->n_shared * L->d_ff_shared;
  w.Hs = L->n_shared ? c.take((size_t)T * Fs * 2) : nullptr;
  w.y_shared = L->n_shared ? (float*)c.take((size_t)T * d * 4) : nullptr;
  w.counts2 = w.offsets2 = w.row_assign2 = w.assign_row2 = nullptr;
  w.lis2 = nullptr;
  m.gidx = (int32_t*)c.take(n * 4);
  m.counts3 = (int32_t*)c.take((size_t)3 * E * 4);
  m.offsets3 = (int32_t*)c.take((size_t)(3 * E + 1) * 4);
  m.row_assign3 = (int32_t*)c.take(n * 4);
  m.assign_row3 = (int32_t*)c.take(n * 4);
  m.gperm_ws = c.take(permute_ws_bytes(T, 3 * E, k));
  m.total = w.total = c.off;
  return m;
}

moe_status check_mwq_groups(const moe_mwq_groups* g) {
  if (!g) return MOE_OK;
  OPT_PTR(g->group_idx, "groups.group_idx");
  OPT_PTR(g->counts, "groups.counts");
  OPT_PTR(g->offsets, "groups.offsets");
  OPT_PTR(g->row_assign, "groups.row_assign");
  OPT_PTR(g->assign_row, "groups.assign_row");
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_mwq_group_workspace_size(int T, int E, int k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  return mwq_group_ws_bytes(T, E, k);
}

moe_status moe_mwq_group(const int32_t* topk_idx, const int32_t* widths, int T, int E, int k,
                         const moe_mwq_groups* out, void* ws, size_t ws_bytes, unsigned flags,
                         void* stream) {
  moe_status s = check_common(T, E, k, flags);
  if (s != MOE_OK) return s;
  if (3 * E > kMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "(expert, width) groups need 3E <= %d (E = %d)", kMaxExperts, E);
  REQUIRE(out, "out must not be NULL");
  s = check_mwq_groups(out);
  if (s != MOE_OK) return s;
  REQUIRE(out->counts && out->offsets, "out->counts and out->offsets must not be NULL");
  if (T > 0) {
    REQUIRE_PTR(topk_idx, "topk_idx");
    REQUIRE_PTR(widths, "widths");
  }
  const size_t need = mwq_group_ws_bytes(T, E, k);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_mwq_group needs %zu workspace bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  REQUIRE(aligned(ws, 256), "ws must be 256-byte aligned");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  hipStream_t st = (hipStream_t)stream;
  const int n = T * k;
  int32_t* gidx = out->group_idx ? out->group_idx : (int32_t*)ws;
  void* pws = (char*)ws + align_up((size_t)n * 4);
  hipError_t e = launch_mwq_group_ids(topk_idx, widths, n, gidx, st);
  if (e != hipSuccess) return hip_status(e, "mwq group ids");
  return hip_status(launch_permute(gidx, T, 3 * E, k, out->counts, out->offsets, out->row_assign,
                                   out->assign_row, nullptr, pws, st),
                    "mwq group permute");
}

size_t moe_grouped_ffn_mwq_workspace_size(int T, int F, int k) {
  if (T < 0 || F < 0 || k < 1) return 0;
  return (size_t)T * k * F * 2;
}

moe_status moe_grouped_ffn_mwq(const void* x, int T, int d, int F, int E, int k, moe_act act,
                               const moe_mwq_experts* w, const int32_t* offsets,
                               const int32_t* row_assign, const float* topk_gate,
                               float* y_rows, void* ws, size_t ws_bytes, unsigned flags,
                               void* stream) {
  moe_status s = check_common(T, E, k, flags);
  if (s != MOE_OK) return s;
  if (3 * E > kMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "(expert, width) groups need 3E <= %d (E = %d)", kMaxExperts, E);
  s = check_mwq_experts(w, T, d, F, k, act);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(offsets, "offsets");
  REQUIRE_PTR(row_assign, "row_assign");
  if (T > 0) REQUIRE_PTR(x, "x");
  REQUIRE_PTR(y_rows, "y_rows");
  OPT_PTR(topk_gate, "topk_gate");
  const size_t need = moe_grouped_ffn_mwq_workspace_size(T, F, k);
  if (need && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "moe_grouped_ffn_mwq needs %zu workspace bytes (got %zu)",
                need, ws ? ws_bytes : (size_t)0);
  OPT_PTR(ws, "ws");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  if (T == 0) return ok();
  MwqProblem p{};
  p.T = T; p.d = d; p.F = F; p.E = E; p.k = k; p.act = act; p.x = x; p.w = w;
  p.offsets = offsets; p.row_assign = row_assign; p.gate = topk_gate; p.y_rows = y_rows;
  p.H = ws; p.rows = T * k;
  return hip_status(launch_mwq_ffn(p, (hipStream_t)stream), "moe_grouped_ffn_mwq launch");
}

moe_status moe_mwq_workspace_size(const moe_layer_desc* L, int T, size_t* bytes) {
  REQUIRE(bytes, "bytes must not be NULL");
  moe_status s = check_layer(L, T, 0, false);
  if (s != MOE_OK) return s;
  *bytes = carve_mwq_layer(L, T, nullptr).total;
  return ok();
}

moe_status moe_layer_forward_mwq(const moe_layer_desc* L, const moe_mwq_experts* W,
                                 const int32_t* widths, const void* x, int T, void* y,
                                 moe_dtype ydt, moe_aux* aux, const moe_mwq_groups* groups,
                                 void* ws, size_t ws_bytes, unsigned flags, void* stream) {
  moe_status s = check_layer(L, T, flags, false);
  if (s != MOE_OK) return s;
  const int E = L->n_experts, k = L->top_k, d = L->d_model, F = L->d_ff;
  if (L->act_dtype != MOE_DT_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "nested experts need bf16 activations");
  if (3 * E > kMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "(expert, width) groups need 3E <= %d (E = %d)", kMaxExperts, E);
  s = check_mwq_experts(W, T, d, F, k, L->act);
  if (s != MOE_OK) return s;
  s = check_mwq_groups(groups);
  if (s != MOE_OK) return s;
  REQUIRE(valid_dtype(ydt), "unknown output dtype %d", (int)ydt);
  if (T > 0) {
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(y, "y");
    REQUIRE_PTR(widths, "widths");
  }
  if (aux) {
    OPT_PTR(aux->logits, "aux.logits"); OPT_PTR(aux->idx, "aux.idx");
    OPT_PTR(aux->gates, "aux.gates"); OPT_PTR(aux->counts, "aux.counts");
    OPT_PTR(aux->offsets, "aux.offsets"); OPT_PTR(aux->row_assign, "aux.row_assign");
    OPT_PTR(aux->assign_row, "aux.assign_row"); OPT_PTR(aux->lis, "aux.lis");
  }
  if ((flags & MOE_F_LOGITS_GIVEN) && !(aux && aux->logits))
    return fail(MOE_ERR_INVALID_ARG, "MOE_F_LOGITS_GIVEN needs aux->logits");
  const size_t need = carve_mwq_layer(L, T, nullptr).total;
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "the layer needs %zu workspace bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  REQUIRE(aligned(ws, 256), "ws must be 256-byte aligned");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  if (T == 0) return ok();

  hipStream_t st = (hipStream_t)stream;
  MwqLayerWs m = carve_mwq_layer(L, T, ws);
  LayerWs& w = m.base;
  float* logits = (aux && aux->logits) ? aux->logits : w.logits;
  int32_t* idx = (aux && aux->idx) ? aux->idx : w.idx;
  float* gates = (aux && aux->gates) ? aux->gates : w.gates;
  int32_t* counts = (aux && aux->counts) ? aux->counts : w.counts;
  int32_t* offsets = (aux && aux->offsets) ? aux->offsets : w.offsets;
  int32_t* row_assign = (aux && aux->row_assign) ? aux->row_assign : w.row_assign;
  int32_t* assign_row = (aux && aux->assign_row) ? aux->assign_row : w.assign_row;
  double* lis = (aux && aux->lis) ? aux->lis : w.lis;
  int32_t* gidx = (groups && groups->group_idx) ? groups->group_idx : m.gidx;
  int32_t* counts3 = (groups && groups->counts) ? groups->counts : m.counts3;
  int32_t* offsets3 = (groups && groups->offsets) ? groups->offsets : m.offsets3;
  int32_t* row_assign3 = (groups && groups->row_assign) ? groups->row_assign : m.row_assign3;
  int32_t* assign_row3 = (groups && groups->assign_row) ? groups->assign_row : m.assign_row3;

  stage(0, st);
  hipError_t e = route_and_permute(L, x, T, logits, idx, gates, counts, offsets, row_assign,
                                   assign_row, lis, w.perm_ws, flags, st);
  if (e != hipSuccess) return hip_status(e, "route and permute");
  e = launch_mwq_group_ids(idx, widths, T * k, gidx, st);
  if (e != hipSuccess) return hip_status(e, "mwq group ids");
  e = launch_permute(gidx, T, 3 * E, k, counts3, offsets3, row_assign3, assign_row3, nullptr,
                     m.gperm_ws, st);
  if (e != hipSuccess) return hip_status(e, "mwq group permute");
  stage(2, st);
  MwqProblem p{};
  p.T = T; p.d = d; p.F = F; p.E = E; p.k = k; p.act = L->act; p.x = x; p.w = W;
  p.offsets = offsets3; p.row_assign = row_assign3; p.gate = gates; p.y_rows = w.y_rows;
  p.H = w.H; p.rows = T * k;
  e = launch_mwq_ffn(p, st, g_stage_on ? g_stage_ev[3] : nullptr);
  if (e != hipSuccess) return hip_status(e, "mwq ffn");
  stage(4, st);
  if (L->n_shared > 0) {
    FfnProblem q{};
    q.T = T; q.d = d; q.F = L->n_shared * L->d_ff_shared; q.E = 1; q.k = 1;
    q.act = MOE_ACT_SWIGLU; q.dt = L->act_dtype; q.x = x; q.w = &L->shared;
    q.offsets = nullptr; q.row_assign = nullptr; q.gate = nullptr;
    q.y_rows = w.y_shared; q.H = w.Hs; q.rows = T;
    e = launch_grouped_ffn(q, st);
    if (e != hipSuccess) return hip_status(e, "shared experts");
  }
  stage(5, st);
  e = launch_combine(w.y_rows, assign_row3, T, k, d, w.y_shared, y, ydt, st);
  stage(6, st);
  return hip_status(e, "combine");
}

}  // extern "C"

// ---- contextual sparse down-projection --------------------------------------

namespace {

moe_status check_floe_experts(const moe_floe_experts* w, int T, int d, int F, int k) {
  REQUIRE(w, "sparse-down experts must not be NULL");
  REQUIRE(w->up, "sparse-down experts: up must not be NULL");
  REQUIRE_PTR(w->up->q2, "up q2");
  REQUIRE(w->up->s2 && w->up->z2, "up s2/z2 must not be NULL");
  REQUIRE(aligned(w->up->s2, 8) && aligned(w->up->z2, 8), "up s2/z2 must be 8-byte aligned");
  REQUIRE_PTR(w->w_gate, "w_gate");
  REQUIRE_PTR(w->w_down_t, "w_down_t");
  REQUIRE_PTR(w->threshold, "threshold");
  if (const char* why = floe_unsupported(T, d, F, k)) return fail(MOE_ERR_UNSUPPORTED, "%s", why);
  return MOE_OK;
}

struct FloeLayerWs {
  LayerWs base;
  float* U;
  uint8_t* flags;
  int32_t *list, *nnz;
  void* Hc;
  size_t total;
};

FloeLayerWs carve_floe_layer(const moe_layer_desc* L, int T, void* ws) {
  const int E = L->n_experts, k = L->top_k, d = L->d_model, F = L->d_ff;
  const size_t n = (size_t)T * k;
  Carver c(ws);
  FloeLayerWs m;
  LayerWs& w = m.base;
  w.logits = (float*)c.take((size_t)T * E * 4);
  w.idx = (int32_t*)c.take(n * 4);
  w.gates = (float*)c.take(n * 4);
  w.counts = (int32_t*)c.take((size_t)E * 4);
  w.offsets = (int32_t*)c.take((size_t)(E + 1) * 4);
  w.row_assign = (int32_t*)c.take(n * 4);
  w.assign_row = (int32_t*)c.take(n * 4);
  w.lis = (double*)c.take(8);
  w.perm_ws = c.take(route_ws_bytes(L, T));
  w.H = nullptr;
  w.down_splits = floe_down_splits(d, E);
  w.y_rows = (float*)c.take(n * d * 4 * w.down_splits);
  const int Fs = L->n_shared * L->d_ff_shared;
  w.Hs = L->n_shared ? c.take((size_t)T * Fs * 2) : nullptr;
  w.y_shared = L->n_shared ? (float*)c.take((size_t)T * d * 4) : nullptr;
  w.counts2 = w.offsets2 = w.row_assign2 = w.assign_row2 = nullptr;
  w.lis2 = nullptr;
  m.U = (float*)c.take(n * F * 4);
  m.flags = (uint8_t*)c.take((size_t)E * F);
  m.list = (int32_t*)c.take((size_t)E * F * 4);
  m.nnz = (int32_t*)c.take((size_t)E * 4);
  m.Hc = c.take(n * F * 2);
  m.total = w.total = c.off;
  return m;
}

}  // namespace

extern "C" {

moe_status moe_floe_workspace_size(const moe_layer_desc* L, int T, size_t* bytes) {
  REQUIRE(bytes, "bytes must not be NULL");
  moe_status s = check_layer(L, T, 0, false);
  if (s != MOE_OK) return s;
  *bytes = carve_floe_layer(L, T, nullptr).total;
  return ok();
}

moe_status moe_layer_forward_floe(const moe_layer_desc* L, const moe_floe_experts* W,
                                  const void* x, int T, void* y, moe_dtype ydt, moe_aux* aux,
                                  const moe_floe_aux* floe_out, void* ws, size_t ws_bytes,
                                  unsigned flags, void* stream) {
  moe_status s = check_layer(L, T, flags, false);
  if (s != MOE_OK) return s;
  const int E = L->n_experts, k = L->top_k, d = L->d_model, F = L->d_ff;
  if (L->act_dtype != MOE_DT_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "sparse-down experts need bf16 activations");
  if (L->act != MOE_ACT_SWIGLU)
    return fail(MOE_ERR_UNSUPPORTED, "sparse-down experts are SwiGLU experts");
  s = check_floe_experts(W, T, d, F, k);
  if (s != MOE_OK) return s;
  REQUIRE(valid_dtype(ydt), "unknown output dtype %d", (int)ydt);
  if (T > 0) {
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(y, "y");
  }
  if (aux) {
    OPT_PTR(aux->logits, "aux.logits"); OPT_PTR(aux->idx, "aux.idx");
    OPT_PTR(aux->gates, "aux.gates"); OPT_PTR(aux->counts, "aux.counts");
    OPT_PTR(aux->offsets, "aux.offsets"); OPT_PTR(aux->row_assign, "aux.row_assign");
    OPT_PTR(aux->assign_row, "aux.assign_row"); OPT_PTR(aux->lis, "aux.lis");
  }
  if (floe_out) {
    OPT_PTR(floe_out->up_out, "floe_out.up_out");
    OPT_PTR(floe_out->kept, "floe_out.kept");
    OPT_PTR(floe_out->channels, "floe_out.channels");
  }
  if ((flags & MOE_F_LOGITS_GIVEN) && !(aux && aux->logits))
    return fail(MOE_ERR_INVALID_ARG, "MOE_F_LOGITS_GIVEN needs aux->logits");
  const size_t need = carve_floe_layer(L, T, nullptr).total;
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "the layer needs %zu workspace bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  REQUIRE(aligned(ws, 256), "ws must be 256-byte aligned");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  if (T == 0) return ok();

  hipStream_t st = (hipStream_t)stream;
  FloeLayerWs m = carve_floe_layer(L, T, ws);
  LayerWs& w = m.base;
  float* logits = (aux && aux->logits) ? aux->logits : w.logits;
  int32_t* idx = (aux && aux->idx) ? aux->idx : w.idx;
  float* gates = (aux && aux->gates) ? aux->gates : w.gates;
  int32_t* counts = (aux && aux->counts) ? aux->counts : w.counts;
  int32_t* offsets = (aux && aux->offsets) ? aux->offsets : w.offsets;
  int32_t* row_assign = (aux && aux->row_assign) ? aux->row_assign : w.row_assign;
  int32_t* assign_row = (aux && aux->assign_row) ? aux->assign_row : w.assign_row;
  double* lis = (aux && aux->lis) ? aux->lis : w.lis;

  stage(0, st);
  hipError_t e = route_and_permute(L, x, T, logits, idx, gates, counts, offsets, row_assign,
                                   assign_row, lis, w.perm_ws, flags, st);
  if (e != hipSuccess) return hip_status(e, "route and permute");
  stage(2, st);
  FloeProblem p{};
  p.T = T; p.d = d; p.F = F; p.E = E; p.k = k; p.x = x; p.w = W; p.offsets = offsets;
  p.row_assign = row_assign; p.gate = gates;
  p.U = (floe_out && floe_out->up_out) ? floe_out->up_out : m.U;
  p.flags = m.flags;
  p.list = (floe_out && floe_out->channels) ? floe_out->channels : m.list;
  p.nnz = (floe_out && floe_out->kept) ? floe_out->kept : m.nnz;
  p.Hc = (u16*)m.Hc;
  p.y_rows = w.y_rows;
  p.rows = T * k;
  p.splits = w.down_splits;
  e = launch_floe_ffn(p, st, g_stage_on ? g_stage_ev[3] : nullptr);
  if (e != hipSuccess) return hip_status(e, "sparse-down ffn");
  stage(4, st);
  if (L->n_shared > 0) {
    FfnProblem q{};
    q.T = T; q.d = d; q.F = L->n_shared * L->d_ff_shared; q.E = 1; q.k = 1;
    q.act = MOE_ACT_SWIGLU; q.dt = L->act_dtype; q.x = x; q.w = &L->shared;
    q.offsets = nullptr; q.row_assign = nullptr; q.gate = nullptr;
    q.y_rows = w.y_shared; q.H = w.Hs; q.rows = T;
    e = launch_grouped_ffn(q, st);
    if (e != hipSuccess) return hip_status(e, "shared experts");
  }
  stage(5, st);
  e = launch_combine(w.y_rows, assign_row, T, k, d, w.y_shared, y, ydt, st, w.down_splits,
                     (size_t)T * k * d);
  stage(6, st);
  return hip_status(e, "combine");
}

}  // extern "C"

// ---- atomic experts on a Cartesian router grid ------------------------------

namespace {

// At most this many tokens, the automatic schedule runs the atomic experts
// expert-centric (when w_out_rows is given): each expert with kept pairs is
// read once, so the layer streams only the experts some token kept, against
// every expert's weights (and a [T][N] matrix) for the dense product.
constexpr int kAtomicEcAutoMaxT = 64;

// The schedule a call runs (MOE_ATOMIC_DENSE or MOE_ATOMIC_EXPERT_CENTRIC), or
// -1 with the error set.
int atomic_schedule(const moe_atomic_layer_desc* L, int T, moe_status* st) {
  *st = MOE_OK;
  const bool ec_ok = L->w_out_rows && atomic_ec_supported(L->d_model);
  switch (L->schedule) {
    case MOE_ATOMIC_DENSE:
      if (!L->w_out) { *st = fail(MOE_ERR_INVALID_ARG, "the dense schedule needs w_out"); return -1; }
      return MOE_ATOMIC_DENSE;
    case MOE_ATOMIC_EXPERT_CENTRIC:
      if (!L->w_out_rows) {
        *st = fail(MOE_ERR_INVALID_ARG, "the expert-centric schedule needs w_out_rows");
        return -1;
      }
      if (!ec_ok) {
        *st = fail(MOE_ERR_UNSUPPORTED,
                   "the expert-centric schedule needs d_model a multiple of 512, at most 4096");
        return -1;
      }
      return MOE_ATOMIC_EXPERT_CENTRIC;
    case MOE_ATOMIC_AUTO:
      if (ec_ok && (T <= kAtomicEcAutoMaxT || !L->w_out)) return MOE_ATOMIC_EXPERT_CENTRIC;
      if (L->w_out) return MOE_ATOMIC_DENSE;
      *st = L->w_out_rows ? fail(MOE_ERR_UNSUPPORTED,
                                 "only w_out_rows given, and the expert-centric schedule needs "
                                 "d_model a multiple of 512, at most 4096")
                          : fail(MOE_ERR_INVALID_ARG, "w_out and w_out_rows are both NULL");
      return -1;
  }
  *st = fail(MOE_ERR_INVALID_ARG, "unknown atomic schedule %d", L->schedule);
  return -1;
}

moe_status check_atomic(const moe_atomic_layer_desc* L, int T, unsigned flags) {
  REQUIRE(L, "layer descriptor must not be NULL");
  REQUIRE((flags & ~kKnownFlags) == 0, "unknown flag bits 0x%x", flags & ~kKnownFlags);
  REQUIRE(!(flags & MOE_F_LOGITS_GIVEN), "MOE_F_LOGITS_GIVEN is not defined for the atomic layer");
  REQUIRE(T >= 0, "T must be >= 0 (got %d)", T);
  const int d = L->d_model, nr = L->grid_rows, nc = L->grid_cols, K = L->top_k;
  REQUIRE(d >= 128 && d % 128 == 0, "atomic layer: d_model must be a positive multiple of 128");
  REQUIRE(nr >= 1 && nc >= 1, "atomic layer: grid must be at least 1 x 1");
  const long long N = (long long)nr * nc;
  REQUIRE(K >= 1 && K <= N, "atomic layer: top_k must be in [1, N] (got %d)", K);
  if (nr > 1024 || nc > 1024 || nc % 32 != 0 || N % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED,
                "atomic layer needs nr, nc <= 1024, nc %% 32 == 0 and N %% 128 == 0 (nr=%d, nc=%d)",
                nr, nc);
  REQUIRE((long long)T * K < (1ll << 31) && (long long)T * N < (1ll << 40), "T too large");
  REQUIRE_PTR(L->w_row, "w_row");
  REQUIRE_PTR(L->w_col, "w_col");
  REQUIRE_PTR(L->w_in, "w_in");
  OPT_PTR(L->w_out, "w_out");
  OPT_PTR(L->w_out_rows, "w_out_rows");
  moe_status st;
  if (atomic_schedule(L, T, &st) < 0) return st;
  REQUIRE(L->n_shared >= 0, "n_shared must be >= 0");
  if (L->n_shared > 0) {
    REQUIRE(L->d_ff_shared >= 8 && L->d_ff_shared % 8 == 0,
            "d_ff_shared must be a positive multiple of 8");
    moe_status s = check_experts(&L->shared, MOE_DT_BF16, d, L->n_shared * L->d_ff_shared,
                                 MOE_ACT_SWIGLU, "shared");
    if (s != MOE_OK) return s;
  }
  return MOE_OK;
}

int atomic_out_splits(int T, int d, int N) {
  const long long tiles = (long long)((T + 255) / 256) * ((d + 255) / 256);
  int S = 1;
  while (tiles * S < 512 && S < 8 && N % (128 * 2 * S) == 0) S *= 2;
  return S;
}

// K slices of the router GEMMs (T x n x d): enough tiles to fill the chip
int atomic_router_splits(int T, int n, int d) {
  const long long tiles = (long long)((T + 255) / 256) * ((n + 255) / 256);
  int S = 1;
  while (tiles * S < 256 && S < 16 && d % (128 * 2 * S) == 0) S *= 2;
  return S;
}

struct AtomicWs {
  float *lr, *lc, *pr, *pc, *gates, *ukept, *y_rows, *y_shared;
  int32_t *idx, *counts, *offsets, *row_assign, *assign_row, *iota, *bitpre;
  uint32_t* bits;
  double* lis;
  void *perm_ws, *H, *Hs;
  void* ec;  // expert-centric schedule: h [T*K] bf16, then the partial sums
  int splits, rsplit, csplit;
  size_t total;
};

// `schedule` as atomic_schedule resolved it; the two schedules carve different
// buffers after the shared routing and grouping ones
AtomicWs carve_atomic(const moe_atomic_layer_desc* L, int T, void* ws, int schedule) {
  const int d = L->d_model, nr = L->grid_rows, nc = L->grid_cols, K = L->top_k;
  const size_t N = (size_t)nr * nc, n = (size_t)T * K, W = N / 32;
  const bool ec = schedule == MOE_ATOMIC_EXPERT_CENTRIC;
  Carver c(ws);
  AtomicWs w;
  w.rsplit = atomic_router_splits(T, nr, d);
  w.csplit = atomic_router_splits(T, nc, d);
  w.lr = (float*)c.take((size_t)w.rsplit * T * nr * 4);
  w.lc = (float*)c.take((size_t)w.csplit * T * nc * 4);
  w.pr = (float*)c.take((size_t)T * nr * 4);
  w.pc = (float*)c.take((size_t)T * nc * 4);
  w.idx = (int32_t*)c.take(n * 4);
  w.gates = (float*)c.take(n * 4);
  w.ukept = (float*)c.take(n * 4);
  w.bits = (uint32_t*)c.take((size_t)T * W * 4);
  w.bitpre = (int32_t*)c.take((size_t)T * W * 4);
  w.counts = (int32_t*)c.take(N * 4);
  w.offsets = (int32_t*)c.take((N + 1) * 4);
  w.row_assign = (int32_t*)c.take(n * 4);
  w.assign_row = (int32_t*)c.take(n * 4);
  w.lis = (double*)c.take(8);
  w.perm_ws = c.take(grid_permute_ws_bytes(T, (int)N));
  w.H = nullptr;
  w.y_rows = nullptr;
  w.iota = nullptr;
  w.ec = nullptr;
  w.splits = 0;
  if (ec) {
    w.ec = c.take(atomic_ec_ws_bytes(T, d, (int)N, K));
  } else {
    w.H = c.take((size_t)T * N * 2);
    w.splits = atomic_out_splits(T, d, (int)N);
    w.y_rows = (float*)c.take((size_t)w.splits * T * d * 4);
    w.iota = (int32_t*)c.take((size_t)T * 4);
  }
  const int Fs = L->n_shared * L->d_ff_shared;
  w.Hs = L->n_shared ? c.take((size_t)T * Fs * 2) : nullptr;
  w.y_shared = L->n_shared ? (float*)c.take((size_t)T * d * 4) : nullptr;
  w.total = c.off;
  return w;
}

}  // namespace

extern "C" {

moe_status moe_atomic_schedule(const moe_atomic_layer_desc* L, int T, int* schedule) {
  REQUIRE(schedule, "schedule must not be NULL");
  moe_status s = check_atomic(L, T, 0);
  if (s != MOE_OK) return s;
  *schedule = atomic_schedule(L, T, &s);
  return ok();
}

moe_status moe_atomic_workspace_size(const moe_atomic_layer_desc* L, int T, size_t* bytes) {
  REQUIRE(bytes, "bytes must not be NULL");
  moe_status s = check_atomic(L, T, 0);
  if (s != MOE_OK) return s;
  *bytes = carve_atomic(L, T, nullptr, atomic_schedule(L, T, &s)).total;
  return ok();
}

moe_status moe_atomic_layer_forward(const moe_atomic_layer_desc* L, const void* x, int T, void* y,
                                    moe_dtype ydt, moe_atomic_aux* aux, void* ws, size_t ws_bytes,
                                    unsigned flags, void* stream) {
  moe_status s = check_atomic(L, T, flags);
  if (s != MOE_OK) return s;
  REQUIRE(valid_dtype(ydt), "unknown output dtype %d", (int)ydt);
  if (T > 0) {
    REQUIRE_PTR(x, "x");
    REQUIRE_PTR(y, "y");
  }
  if (aux) {
    OPT_PTR(aux->logp_row, "aux.logp_row"); OPT_PTR(aux->logp_col, "aux.logp_col");
    OPT_PTR(aux->idx, "aux.idx"); OPT_PTR(aux->gates, "aux.gates");
    OPT_PTR(aux->counts, "aux.counts"); OPT_PTR(aux->offsets, "aux.offsets");
    OPT_PTR(aux->row_assign, "aux.row_assign"); OPT_PTR(aux->assign_row, "aux.assign_row");
    OPT_PTR(aux->lis, "aux.lis");
  }
  const int sched = atomic_schedule(L, T, &s);
  const size_t need = carve_atomic(L, T, nullptr, sched).total;
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "the atomic layer needs %zu workspace bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  REQUIRE(aligned(ws, 256), "ws must be 256-byte aligned");
  if (flags & MOE_F_VALIDATE_ONLY) return ok();
  if (T == 0) return ok();

  hipStream_t st = (hipStream_t)stream;
  AtomicWs w = carve_atomic(L, T, ws, sched);
  const int d = L->d_model, nr = L->grid_rows, nc = L->grid_cols, K = L->top_k;
  const int N = nr * nc;
  float* pr = (aux && aux->logp_row) ? aux->logp_row : w.pr;
  float* pc = (aux && aux->logp_col) ? aux->logp_col : w.pc;
  int32_t* idx = (aux && aux->idx) ? aux->idx : w.idx;
  float* gates = (aux && aux->gates) ? aux->gates : w.gates;
  int32_t* counts = (aux && aux->counts) ? aux->counts : w.counts;
  int32_t* offsets = (aux && aux->offsets) ? aux->offsets : w.offsets;
  int32_t* row_assign = (aux && aux->row_assign) ? aux->row_assign : w.row_assign;
  int32_t* assign_row = (aux && aux->assign_row) ? aux->assign_row : w.assign_row;
  double* lis = (aux && aux->lis) ? aux->lis : w.lis;
  const u16* X = (const u16*)x;

  stage(0, st);
  const size_t sr = (size_t)T * nr, sc = (size_t)T * nc;
  hipError_t e = launch_gemm_bt(X, d, T, (const u16*)L->w_row, nr, d, w.lr, w.rsplit, sr, st);
  if (e == hipSuccess)
    e = launch_gemm_bt(X, d, T, (const u16*)L->w_col, nc, d, w.lc, w.csplit, sc, st);
  if (e == hipSuccess) e = launch_log_softmax_rows(w.lr, T, nr, pr, st, w.rsplit, sr);
  if (e == hipSuccess) e = launch_log_softmax_rows(w.lc, T, nc, pc, st, w.csplit, sc);
  if (e == hipSuccess)
    e = launch_grid_topk(pr, pc, T, nr, nc, K, idx, gates, w.bits, w.bitpre, st);
  if (e != hipSuccess) return hip_status(e, "grid routing");
  stage(1, st);
  e = launch_grid_permute(w.bits, w.bitpre, T, N, K, counts, offsets, row_assign, assign_row, lis,
                          w.perm_ws, st);
  if (e != hipSuccess) return hip_status(e, "grid permutation");
  stage(2, st);
  const bool ec = sched == MOE_ATOMIC_EXPERT_CENTRIC;
  u16* hrow = ec ? (u16*)w.ec : nullptr;
  float* ypart = ec ? (float*)((char*)w.ec + align_up((size_t)T * K * 2)) : nullptr;
  if (ec) {
    // expert-centric: each expert with kept pairs reads its w_in / w_out once
    e = launch_atomic_ec_in(X, T, d, (const u16*)L->w_in, N, offsets, row_assign, gates, K, hrow,
                            st);
    if (e != hipSuccess) return hip_status(e, "atomic expert-centric input");
    stage(3, st);
    e = launch_atomic_ec_out(hrow, offsets, row_assign, K, (const u16*)L->w_out_rows, N, d, T,
                             ypart, st);
    if (e != hipSuccess) return hip_status(e, "atomic expert-centric output");
  } else {
    e = launch_atomic_in(X, T, (const u16*)L->w_in, N, d, w.bits, w.bitpre, idx, gates, K,
                         w.ukept, (u16*)w.H, st);
    if (e != hipSuccess) return hip_status(e, "atomic input GEMM");
    stage(3, st);
    e = launch_gemm_bt((const u16*)w.H, N, T, (const u16*)L->w_out, d, N, w.y_rows, w.splits,
                       (size_t)T * d, st);
    if (e != hipSuccess) return hip_status(e, "atomic output GEMM");
  }
  stage(4, st);
  if (L->n_shared > 0) {
    FfnProblem q{};
    q.T = T; q.d = d; q.F = L->n_shared * L->d_ff_shared; q.E = 1; q.k = 1;
    q.act = MOE_ACT_SWIGLU; q.dt = MOE_DT_BF16; q.x = x; q.w = &L->shared;
    q.offsets = nullptr; q.row_assign = nullptr; q.gate = nullptr;
    q.y_rows = w.y_shared; q.H = w.Hs; q.rows = T;
    e = launch_grouped_ffn(q, st);
    if (e != hipSuccess) return hip_status(e, "shared experts");
  }
  stage(5, st);
  if (ec) {
    e = launch_atomic_ec_reduce(ypart, T, d, N, w.y_shared, y, ydt, st);
  } else {
    e = launch_iota(w.iota, T, st);
    if (e == hipSuccess)
      e = launch_combine(w.y_rows, w.iota, T, 1, d, w.y_shared, y, ydt, st, w.splits,
                         (size_t)T * d);
  }
  stage(6, st);
  return hip_status(e, "combine");
}

}  // extern "C"
