/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer forward.
 *
 * The layer, in the order the calls below run it:
 *   1. router logits and top-k expert selection per token, with softmax gate
 *      weights over the selected k ........................... moe_route_topk
 *   2. expert-centric permutation: per-expert token counts, offsets, a stable
 *      expert-major row order, and the Load Imbalance Score .. moe_permute
 *   3. grouped expert FFN (SwiGLU or ReLU; bf16, fp32 or group-wise INT4
 *      weights decoded inside the GEMM), gate-scaled rows .... moe_grouped_ffn
 *   4. weighted combine back to token order (+ shared experts)  moe_combine
 *   moe_layer_forward chains 1-4 (and the always-active shared experts).
 *
 * Sources (page title -- section):
 *   "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale" --
 *     Core claim, What carries the argument, Figure 3 (expert-centric
 *     scheduling: group active experts contiguously, run each group as a
 *     grouped GEMM); Axiom ledger (exact top-K); abstract and Figure 1 (a shared
 *     dense branch that is always active).
 *   "A Replicate-and-Quantize Strategy for Plug-and-Play Load Balancing of
 *     Sparse Mixture-of-Experts LLMs" -- What carries the argument, and
 *     Definition 1 quoted in its Circularity Check (n_j tokens routed to expert
 *     j; LIS = m * max_j n_j / (n * k)).
 *   "FloE: On-the-Fly MoE Inference on Memory-constrained GPU" -- What carries
 *     the argument, Core claim, Figure 11 (expert = W_gate, W_up, W_down, SiLU on
 *     the gate projection, up output feeding the down projection).
 *   "D^2MoE: Dual Routing and Dynamic Scheduling for Efficient On-Device
 *     MoE-based LLM Serving" -- What carries the argument (asymmetric
 *     quantisation), Assumptions & free parameters (group size 128), Figure 8
 *     (dequantisation fused into the GEMM kernel).
 *
 * Conventions shared by every call:
 *   - Array arguments are DEVICE pointers owned by the caller, row-major, at
 *     least 16-byte aligned.  They must stay valid until the enqueued work
 *     completes.  The library allocates no memory.
 *   - Every call enqueues on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns without synchronising the host.  Nothing is read back.
 *   - Arguments are checked on the host before anything is enqueued: a call
 *     that returns an error has enqueued nothing.  Faults inside kernels show
 *     up at the caller's next synchronisation.  MOE_F_VALIDATE_ONLY runs the
 *     checks and returns without touching the device (usable with no GPU).
 *   - T = 0 is a no-op returning MOE_OK (moe_permute then writes LIS = NaN).
 *   - Limits: 1 <= E <= 64, 1 <= k <= min(E, 8), d and d_ff multiples of 8
 *     (multiples of 128 along K for INT4).  Out-of-range shapes return
 *     MOE_ERR_INVALID_ARG, in-range but unimplemented ones MOE_ERR_UNSUPPORTED.
 *   - Routing, counts, permutation and LIS are exact integer results.  All
 *     outputs are bitwise run-to-run deterministic (MOE_F_NONDETERMINISTIC_COMBINE
 *     is reserved: accepted and ignored).
 *   - The library is stateless apart from a device-property cache and a
 *     thread-local error string; calls are thread-safe.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad shape, misalignment, bad flag */
  MOE_ERR_UNSUPPORTED = 2, /* valid request this build does not implement */
  MOE_ERR_WORKSPACE = 3,   /* ws == NULL or ws_bytes below the size query */
  MOE_ERR_HIP = 4          /* a HIP runtime call failed (launch, device query) */
} moe_status;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype;
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU = 1 } moe_act;

enum {
  MOE_F_LOGITS_GIVEN = 1u,   /* moe_route_topk / layer: `logits` is an input */
  MOE_F_VALIDATE_ONLY = 2u,  /* check arguments, enqueue nothing */
  MOE_F_NONDETERMINISTIC_COMBINE = 4u, /* reserved: accepted and ignored; every path is
                                          deterministic (the fused combine of decode
                                          layers adds at most two rows onto a zeroed
                                          output, which gives the same sum in either
                                          order) */
  MOE_F_BF16_ROWS = 8u /* layer calls with bf16 activations on the tiled path (T > 64,
                          dense experts, d_ff a multiple of 128): the gate-scaled expert
                          rows between the down pass and the combine are stored as bf16
                          (RNE) instead of fp32, halving that traffic (the k rows per
                          token of k = 6 layers); each row then carries one more bf16
                          rounding before the fixed-order fp32 sum.  Ignored elsewhere
                          (weight streaming writes y directly or keeps fp32 rows). */
};

/* Group-wise asymmetric INT4 weights of one projection, all experts.
 * Logical weight W[e][n][kk] (n = output row, kk along the reduction K):
 *   q     : int32 [E][N][K/8]; nibble i (bits 4i..4i+3) of word j holds kk = 8j+i
 *   scale : fp16 bits [E][N][K/128]
 *   zero  : fp16 bits [E][N][K/128]
 * decoded as W = bf16_RNE( fp32( fp32(q) - fp32(zero) ) * fp32(scale) ), each
 * fp32 operation rounded to nearest even, group g = kk / 128. */
typedef struct {
  const int32_t* q;
  const uint16_t* scale;
  const uint16_t* zero;
} moe_w4;

/* Expert weights.  Dense: w_gate, w_up [E][F][d], w_down [E][d][F] in `dtype`.
 * ReLU experts use w_up as W_in and leave w_gate NULL.  If q_up is non-NULL the
 * INT4 form is used (q_gate, q_up with N = F, K = d; q_down with N = d, K = F)
 * and the dense pointers are ignored; INT4 requires bf16 activations. */
typedef struct {
  moe_dtype dtype;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const moe_w4* q_gate;
  const moe_w4* q_up;
  const moe_w4* q_down;
} moe_experts;

/* One MoE layer.  w_router [E][d] in act_dtype, b_router [E] fp32 or NULL.
 * Shared experts (n_shared > 0): SwiGLU, weight 1 on every token, given as one
 * concatenated expert of d_ff = n_shared * d_ff_shared (shared.w_gate/w_up
 * [n_shared*d_ff_shared][d], shared.w_down [d][n_shared*d_ff_shared]); they do
 * not enter routing, counts or LIS. */
typedef struct {
  int d_model, d_ff, n_experts, top_k;
  moe_act act;
  moe_dtype act_dtype;
  const void* w_router;
  const float* b_router;
  moe_experts routed;
  int n_shared, d_ff_shared;
  moe_experts shared;
} moe_layer_desc;

/* Optional outputs of moe_layer_forward; every pointer may be NULL (the
 * workspace then holds the value).  Shapes as in the individual calls. */
typedef struct {
  float* logits;      /* [T][E] (input when MOE_F_LOGITS_GIVEN) */
  int32_t* idx;       /* [T][k] */
  float* gates;       /* [T][k] */
  int32_t* counts;    /* [E] */
  int32_t* offsets;   /* [E+1] */
  int32_t* row_assign;/* [T*k] */
  int32_t* assign_row;/* [T*k] */
  double* lis;        /* [1] */
} moe_aux;

/* Router logits and exact top-k (OmniMoE -- Core claim; Axiom ledger).
 *   x        [T][d] in xdt;  w_router [E][d] in xdt;  b_router [E] fp32 or NULL
 *   logits   [T][E] fp32: written = fp32(x . w_router[e] + b[e]); with
 *            MOE_F_LOGITS_GIVEN it is read instead and x / w_router may be NULL
 *   topk_idx [T][k] int32: slot 0 holds the largest logit; ties go to the lower
 *            expert id; -0.0 and +0.0 compare equal
 *   topk_gate[T][k] fp32: softmax over the k selected logits (sums to 1; k = 1
 *            gives exactly 1).  May be NULL.
 * Logits must be finite; non-finite logits give an unspecified selection. */
moe_status moe_route_topk(const void* x, moe_dtype xdt, const void* w_router,
                          const float* b_router, int T, int d, int E, int k, float* logits,
                          int32_t* topk_idx, float* topk_gate, unsigned flags, void* stream);

/* Expert-centric permutation and load statistics (OmniMoE -- What carries the
 * argument, Figure 3; Replicate-and-Quantize -- Definition 1).
 *   topk_idx   [T][k] int32, each in [0, E)  (flat assignment a = t*k + j)
 *   counts     [E]   n_e = #{a : topk_idx[a] = e}
 *   offsets    [E+1] exclusive prefix of counts (offsets[E] = T*k)
 *   row_assign [T*k] row -> a, rows grouped by expert, a ascending in a group
 *   assign_row [T*k] a -> row (inverse of row_assign)
 *   lis        [1]   fp64: E * max_e n_e / (T * k), NaN for T = 0
 * Any output except counts/offsets may be NULL.  Workspace: at least
 * moe_permute_workspace_size(T, E, k) bytes. */
moe_status moe_permute(const int32_t* topk_idx, int T, int E, int k, int32_t* counts,
                       int32_t* offsets, int32_t* row_assign, int32_t* assign_row, double* lis,
                       void* ws, size_t ws_bytes, unsigned flags, void* stream);
size_t moe_permute_workspace_size(int T, int E, int k);

/* Grouped expert FFN over expert-major rows (FloE -- What carries the argument,
 * Figure 11; OmniMoE -- Figure 3; D^2MoE -- Figure 8 for the INT4 form).
 * Row r of expert e (offsets[e] <= r < offsets[e+1]) is token
 * t = row_assign[r] / k; its output is
 *   y_rows[r] = gate(r) * W_down[e] . h,   h = silu(W_gate[e] x_t) * (W_up[e] x_t)
 *   (ReLU: h = max(0, W_in[e] x_t)), h rounded to bf16 for bf16 activations,
 * with gate(r) = topk_gate[row_assign[r]] (1 if topk_gate is NULL).
 *   x [T][d] in xdt; offsets NULL means one expert covering all T rows with
 *   E = 1 and k = 1; row_assign NULL means row r is token r; y_rows [T*k][d] fp32.
 * Workspace: moe_grouped_ffn_workspace_size(T, d, F, E, k, act, w) bytes. */
moe_status moe_grouped_ffn(const void* x, moe_dtype xdt, int T, int d, int F, int E, int k,
                           moe_act act, const moe_experts* w, const int32_t* offsets,
                           const int32_t* row_assign, const float* topk_gate, float* y_rows,
                           void* ws, size_t ws_bytes, unsigned flags, void* stream);
size_t moe_grouped_ffn_workspace_size(int T, int d, int F, int E, int k, moe_act act,
                                      const moe_experts* w);

/* Weighted combine back to token order.  y_rows hold gate-scaled rows:
 *   y[t][i] = sum_{j<k} y_rows[assign_row[t*k+j]][i] (+ y_shared[t][i])
 * summed in slot order j = 0..k-1, then the shared term.  y in ydt (fp32 or
 * bf16 RNE); y_shared [T][d] fp32 or NULL. */
moe_status moe_combine(const float* y_rows, const int32_t* assign_row, int T, int k, int d,
                       const float* y_shared, void* y, moe_dtype ydt, unsigned flags,
                       void* stream);

/* The whole layer: route, permute, grouped FFN, shared experts, combine.
 *   x [T][d] in L->act_dtype;  y [T][d] in ydt;  aux optional (see moe_aux).
 * Workspace: moe_workspace_size(L, T, &bytes). */
moe_status moe_layer_forward(const moe_layer_desc* L, const void* x, int T, void* y,
                             moe_dtype ydt, moe_aux* aux, void* ws, size_t ws_bytes,
                             unsigned flags, void* stream);

/* Workspace bytes moe_layer_forward needs for T tokens (host only, pure). */
moe_status moe_workspace_size(const moe_layer_desc* L, int T, size_t* bytes);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, arithmetic and results as
 * moe_layer_forward.  The workspace is a static device array of
 * moe_noalloc_scratch_bytes() bytes (64 MiB) that every GPU the library runs
 * on holds until the process ends; its address is looked up once per device
 * on the first call there.  The call allocates nothing.
 *   - A call whose workspace (moe_workspace_size) exceeds the array returns
 *     MOE_ERR_WORKSPACE and enqueues nothing (decode-sized calls fit: at the
 *     Mixtral shape, T up to a few hundred tokens).
 *   - Every call on one GPU uses that GPU's one array, which keeps the last
 *     call's contents; nothing in it has to start at zero (each call writes
 *     what it reads).  Calls whose work overlaps on one GPU (other streams,
 *     other threads) race on it: the caller serialises them. */
moe_status moe_layer_forward_noalloc(const moe_layer_desc* L, const void* x, int T, void* y,
                                     moe_dtype ydt, moe_aux* aux, unsigned flags, void* stream);
/* Bytes of the static array behind moe_layer_forward_noalloc (host only). */
size_t moe_noalloc_scratch_bytes(void);

/* ---- Replica of the heaviest-loaded expert ("A Replicate-and-Quantize
 * Strategy for Plug-and-Play Load Balancing of Sparse Mixture-of-Experts
 * LLMs" -- What carries the argument: a quantized copy of the heavy-hitter
 * expert is appended to the layer, the router left unchanged).  The pages do
 * not say how that expert's tokens reach the copy; this library's rule: its
 * assignments, in flat order a = t*k + j, alternate -- even ranks stay with
 * the expert, odd ranks go to the replica, which is slot E.  Counts, offsets,
 * the permutation and LIS are then those of the split routing over E + 1
 * slots (LIS with m = E + 1). */

/* The replica: INT4 weights of one expert (same layout as moe_w4 with E = 1:
 * q_gate, q_up [1][d_ff][d_model/8], q_down [1][d_model][d_ff/8]; q_gate NULL
 * for ReLU layers) and the expert it copies. */
typedef struct {
  int expert;
  const moe_w4* q_gate;
  const moe_w4* q_up;
  const moe_w4* q_down;
} moe_replica;

/* Remap a permutation (the outputs of moe_permute for topk_idx) to the split
 * routing of expert `heavy`: idx_out [T][k] (heavy's odd-ranked assignments
 * become E), counts_out [E+1], offsets_out [E+2], row_assign_out and
 * assign_row_out [T*k], lis_out [1].  Every output may be NULL.  Equal to
 * moe_permute of idx_out over E+1 slots, without a second sort. */
moe_status moe_replica_split(const int32_t* topk_idx, const int32_t* counts,
                             const int32_t* offsets, const int32_t* assign_row, int T, int E,
                             int k, int heavy, int32_t* idx_out, int32_t* counts_out,
                             int32_t* offsets_out, int32_t* row_assign_out,
                             int32_t* assign_row_out, double* lis_out, unsigned flags,
                             void* stream);

/* The layer with the replica: route, permute, split, grouped FFN of experts
 * 0..E-1 (their own weights) and of slot E (the replica's INT4 weights),
 * shared experts, combine.  bf16 activations only.  aux (optional) receives
 * the split routing: counts [E+1], offsets [E+2], row_assign/assign_row, lis
 * over E+1 slots (aux->idx keeps the router's choice); lis_base (optional)
 * receives the LIS of the router's own routing (E slots).
 * Workspace: moe_replica_workspace_size(L, T, &bytes). */
moe_status moe_layer_forward_replica(const moe_layer_desc* L, const moe_replica* R,
                                     const void* x, int T, void* y, moe_dtype ydt, moe_aux* aux,
                                     double* lis_base, void* ws, size_t ws_bytes, unsigned flags,
                                     void* stream);
moe_status moe_replica_workspace_size(const moe_layer_desc* L, int T, size_t* bytes);

/* ---- Nested (matryoshka) low-bit experts ("D^2MoE: Dual Routing and Dynamic
 * Scheduling for Efficient On-Device MoE-based LLM Serving" -- What carries the
 * argument: one stored copy of each expert serves several bit widths, the
 * lower-bit weights nested inside the higher-bit ones; Assumptions & free
 * parameters: group size 128).  The pages fix the nesting, not the residual's
 * form; this library's format: an asymmetric INT2 base per group of 128 along K,
 * and for width 3 and 4 one binary residual plane each, a bit per weight and an
 * fp16 magnitude per group.  At width b (2, 3 or 4) the weight is
 *   w = fp32( fp32(q) - z2 ) * s2              (each fp32 operation rounded to
 *   b >= 3: w = w + (r3 ? a3 : -a3)             nearest even, no fused
 *   b == 4: w = w + (r4 ? a4 : -a4)             multiply-add)
 *   W = bf16_RNE(w)
 * Every (token, slot) assignment carries its own width, so an expert's rows are
 * grouped by (expert, width): group v = 3*e + (width - 2), 3E groups. */

/* One projection of all experts in the nested format, N output rows and K along
 * the reduction (K a multiple of 128), every pointer non-NULL (q2, p3, p4
 * 16-byte aligned; s2, z2, a3, a4 8-byte aligned):
 *   q2     int32 [E][N][K/16]: word j holds the 2-bit codes of K-indices
 *          16j..16j+15, byte-transposed -- K-index 16j + 4m + b (m, b < 4) in
 *          bits 8b+2m .. 8b+2m+1;
 *   s2, z2 fp16 bits [E][N][K/128]: base scale and zero point;
 *   p3, p4 int32 [E][N][K/32]: residual bits; word j covers K-indices
 *          32j..32j+31, K-index 32j + 4i + b (i < 8, b < 4) in bit 8b + i;
 *   a3, a4 fp16 bits [E][N][K/128]: residual magnitudes.
 * The byte-transposed order puts, after one shift and mask, the codes of four
 * consecutive weights in the four bytes of a word. */
typedef struct {
  const int32_t* q2;
  const uint16_t* s2;
  const uint16_t* z2;
  const int32_t* p3;
  const uint16_t* a3;
  const int32_t* p4;
  const uint16_t* a4;
} moe_wmwq;

/* Nested experts: gate and up with N = d_ff, K = d_model; down with N = d_model,
 * K = d_ff.  ReLU experts use `up` as W_in and leave `gate` NULL. */
typedef struct {
  const moe_wmwq* gate;
  const moe_wmwq* up;
  const moe_wmwq* down;
} moe_mwq_experts;

/* Optional outputs of the (expert, width) grouping; every pointer may be NULL. */
typedef struct {
  int32_t* group_idx;  /* [T][k] 3*topk_idx + (width - 2) */
  int32_t* counts;     /* [3E] rows per group */
  int32_t* offsets;    /* [3E+1] exclusive prefix */
  int32_t* row_assign; /* [T*k] row -> flat assignment, groups in order, a ascending */
  int32_t* assign_row; /* [T*k] inverse */
} moe_mwq_groups;

/* Group the assignments by (expert, width): moe_permute of
 * group_idx = 3*topk_idx + (clamp(widths, 2, 4) - 2) over 3E groups.
 *   topk_idx, widths [T][k] int32 (a width outside 2..4 is clamped to it);
 *   outputs as in moe_mwq_groups (counts and offsets required).
 * 3E <= 64.  Workspace: moe_mwq_group_workspace_size(T, E, k) bytes. */
moe_status moe_mwq_group(const int32_t* topk_idx, const int32_t* widths, int T, int E, int k,
                         const moe_mwq_groups* out, void* ws, size_t ws_bytes, unsigned flags,
                         void* stream);
size_t moe_mwq_group_workspace_size(int T, int E, int k);

/* Grouped expert FFN on nested weights, rows grouped by (expert, width) as
 * moe_mwq_group leaves them: row r with offsets[3e+j] <= r < offsets[3e+j+1]
 * runs expert e decoded at width 2 + j; otherwise as moe_grouped_ffn (bf16
 * activations; y_rows [T*k][d] fp32, gate-scaled).  d_model and d_ff must be
 * multiples of 512.  Workspace: moe_grouped_ffn_mwq_workspace_size(T, F, k). */
moe_status moe_grouped_ffn_mwq(const void* x, int T, int d, int F, int E, int k, moe_act act,
                               const moe_mwq_experts* w, const int32_t* offsets,
                               const int32_t* row_assign, const float* topk_gate,
                               float* y_rows, void* ws, size_t ws_bytes, unsigned flags,
                               void* stream);
size_t moe_grouped_ffn_mwq_workspace_size(int T, int F, int k);

/* The layer with nested routed experts: route, permute (aux: the router's own
 * routing over E experts, as moe_layer_forward), group by (expert, width)
 * (groups, optional), nested FFN, shared experts (dense, from L->shared),
 * combine.  L->routed is not read; bf16 activations only.  widths [T][k] int32
 * gives the width of each assignment.
 * Workspace: moe_mwq_workspace_size(L, T, &bytes). */
moe_status moe_layer_forward_mwq(const moe_layer_desc* L, const moe_mwq_experts* W,
                                 const int32_t* widths, const void* x, int T, void* y,
                                 moe_dtype ydt, moe_aux* aux, const moe_mwq_groups* groups,
                                 void* ws, size_t ws_bytes, unsigned flags, void* stream);
moe_status moe_mwq_workspace_size(const moe_layer_desc* L, int T, size_t* bytes);

/* ---- Contextual sparse down-projection ("FloE: On-the-Fly MoE Inference on
 * Memory-constrained GPU" -- Core claim, What carries the argument; Assumptions
 * & free parameters: one threshold per expert from the empirical distribution
 * of activations).  Per (token, expert) row, with u = W_up x (INT2 up weights,
 * fp32 accumulate), channel f is kept when |u_f| > threshold[e]; then
 *   h_f = kept ? bf16_RNE( silu(W_gate[f] . x) * u_f ) : 0,   y_row = W_down h,
 * so gate rows and down columns of pruned channels are never read. */

/* Sparse-down experts (bf16 activations, SwiGLU):
 *   up        INT2 up projection: q2, s2, z2 of moe_wmwq (N = d_ff, K = d_model,
 *             decoded as the nested format at width 2); p3, a3, p4, a4 unused
 *   w_gate    bf16 [E][d_ff][d_model]
 *   w_down_t  bf16 [E][d_ff][d_model]: W_down transposed, row f holds the
 *             down-projection column of channel f
 *   threshold fp32 [E] */
typedef struct {
  const moe_wmwq* up;
  const void* w_gate;
  const void* w_down_t;
  const float* threshold;
} moe_floe_experts;

/* Optional outputs of moe_layer_forward_floe; every pointer may be NULL. */
typedef struct {
  float* up_out;      /* [T*k][d_ff] fp32 u of each row, rows expert-major */
  int32_t* kept;      /* [E] channels some row of the expert keeps */
  int32_t* channels;  /* [E][d_ff] those channels ascending (first kept[e]) */
} moe_floe_aux;

/* The layer with sparse-down routed experts: route, permute (aux as in
 * moe_layer_forward), INT2 up projection, per-expert kept channels, gate rows
 * and down columns of kept channels only, shared experts (dense, L->shared),
 * combine.  L->routed is not read.  Requires bf16 activations, SwiGLU, d_model
 * and d_ff multiples of 512.  Workspace: moe_floe_workspace_size(L, T, &bytes). */
moe_status moe_layer_forward_floe(const moe_layer_desc* L, const moe_floe_experts* W,
                                  const void* x, int T, void* y, moe_dtype ydt, moe_aux* aux,
                                  const moe_floe_aux* floe_out, void* ws, size_t ws_bytes,
                                  unsigned flags, void* stream);
moe_status moe_floe_workspace_size(const moe_layer_desc* L, int T, size_t* bytes);

/* ---- Atomic experts on a Cartesian router grid ("OmniMoE: An Efficient MoE by
 * Orchestrating Atomic Experts at Scale" -- What carries the argument, Core
 * claim; Axiom ledger: the selection is the exact global top-K).  Expert
 * n = i*nc + j is cell (i, j) of an nr x nc grid and one vector pair
 * (w_in[n], w_out[:, n]).  Per token:
 *   lr = x W_row^T, lc = x W_col^T (fp32), pr = log_softmax(lr), pc = log_softmax(lc)
 *   S_n = fp32(pr[i] + pc[j]); the K cells with the largest S (equal S: lower n)
 *   are kept, slots in ascending n; gates g = softmax over the kept S
 *   y = sum over kept n of w_out[:, n] * bf16_RNE(g_n * silu(x . w_in[n]))
 *       + the shared SwiGLU MLP (n_shared > 0)
 * The kept (token, expert) pairs are grouped by expert (counts, offsets,
 * token-ordered rows, LIS = N * max_n count_n / (T * K)). */
/* How the kept pairs are executed (OmniMoE -- What carries the argument,
 * Figure 3: expert-centric scheduling).  Both give the same result within
 * floating-point summation order.
 *   MOE_ATOMIC_DENSE: one dense GEMM of x against all N input vectors whose
 *     epilogue keeps only the kept cells (gate and SiLU applied, rounded to
 *     bf16, zeros elsewhere), then one dense GEMM of that [T][N] matrix against
 *     w_out.  Needs w_out.  At 4096 tokens every block of 256 consecutive
 *     experts is kept by nearly every token, so this is the grouped product of
 *     each expert group with its tokens, run as MFMA tiles.
 *   MOE_ATOMIC_EXPERT_CENTRIC: the grouping drives the compute: each expert
 *     with kept pairs reads w_in[n] once for all of its tokens, then w_out[n]
 *     (from w_out_rows) once, adding h * w_out[n] into per-range partial sums
 *     that are added in range order; experts no token kept are never read.
 *     Needs w_out_rows and d_model a multiple of 512, at most 4096.
 *   MOE_ATOMIC_AUTO: expert-centric for at most 64 tokens when w_out_rows is
 *     given (or when w_out is NULL), dense otherwise. */
enum { MOE_ATOMIC_AUTO = 0, MOE_ATOMIC_DENSE = 1, MOE_ATOMIC_EXPERT_CENTRIC = 2 };

typedef struct {
  int d_model;
  int grid_rows, grid_cols;  /* nr, nc: N = nr * nc atomic experts */
  int top_k;                 /* K */
  const void* w_row;         /* bf16 [nr][d_model] */
  const void* w_col;         /* bf16 [nc][d_model] */
  const void* w_in;          /* bf16 [N][d_model] */
  const void* w_out;         /* bf16 [d_model][N]: column n is w_out of expert n (dense
                                schedule); may be NULL */
  int n_shared, d_ff_shared;
  moe_experts shared;        /* as in moe_layer_desc */
  const void* w_out_rows;    /* bf16 [N][d_model]: row n is w_out of expert n, the same
                                values expert-major (expert-centric schedule); may be NULL */
  int schedule;              /* MOE_ATOMIC_AUTO, MOE_ATOMIC_DENSE or MOE_ATOMIC_EXPERT_CENTRIC */
} moe_atomic_layer_desc;

/* Optional outputs of moe_atomic_layer_forward; every pointer may be NULL. */
typedef struct {
  float* logp_row;      /* [T][nr] */
  float* logp_col;      /* [T][nc] */
  int32_t* idx;         /* [T][K] kept experts, ascending */
  float* gates;         /* [T][K] */
  int32_t* counts;      /* [N] */
  int32_t* offsets;     /* [N+1] */
  int32_t* row_assign;  /* [T*K] row -> flat pair t*K + slot, experts in order */
  int32_t* assign_row;  /* [T*K] */
  double* lis;          /* [1] */
} moe_atomic_aux;

/* The atomic-expert layer.  x [T][d_model] bf16, y [T][d_model] in ydt.
 * Requires d_model % 128 == 0, nc % 32 == 0, nr, nc <= 1024, N % 128 == 0,
 * 1 <= K <= N; the schedule's own needs are listed with moe_atomic_layer_desc
 * (unmet: MOE_ERR_INVALID_ARG for a missing matrix, MOE_ERR_UNSUPPORTED for
 * d_model).  Workspace: moe_atomic_workspace_size (it depends on the schedule
 * the call resolves to). */
moe_status moe_atomic_layer_forward(const moe_atomic_layer_desc* L, const void* x, int T, void* y,
                                    moe_dtype ydt, moe_atomic_aux* aux, void* ws, size_t ws_bytes,
                                    unsigned flags, void* stream);
moe_status moe_atomic_workspace_size(const moe_atomic_layer_desc* L, int T, size_t* bytes);
/* The schedule (MOE_ATOMIC_DENSE or MOE_ATOMIC_EXPERT_CENTRIC) a call of the
 * atomic layer with T tokens runs (host only, pure; errors as the layer's). */
moe_status moe_atomic_schedule(const moe_atomic_layer_desc* L, int T, int* schedule);

/* Instrumentation (not part of the layer's arithmetic).  While set, every
 * moe_layer_forward call made on this thread records events[i] (hipEvent_t
 * handles created by the caller) on its stream at the stage boundaries:
 *   0 start, 1 after routing, 2 after permutation, 3 after the gate/up GEMM,
 *   4 after the down GEMM, 5 after the shared experts, 6 after the combine.
 * n must be 7; events == NULL turns recording off.  The events let a caller
 * time each stage on the launch stream without a profiler. */
moe_status moe_set_stage_events(void* const* events, int n);

const char* moe_status_string(moe_status s);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
