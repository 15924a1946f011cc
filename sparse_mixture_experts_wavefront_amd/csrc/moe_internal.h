// moe_internal.h -- device helpers and kernel launchers shared by the HIP
// translation units of libmoe.so.  Not installed, not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxExperts = 64;
constexpr int kMaxTopK = 8;
constexpr int kPermChunk = 2048;      // assignments per block in the multi-block permutation
constexpr int kPermFusedMax = 2048;  // up to this many assignments: one fused block
constexpr int kPermFusedBigMax = 8192;  // up to this many: one 1024-thread block

__device__ __forceinline__ float bf16_to_f32(u16 b) {
  return __uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ u16 f32_to_bf16(float f) {  // RNE (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(u16, (__bf16)f);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ float h2f(u16 h) { return (float)__builtin_bit_cast(_Float16, h); }
// two fp32 -> packed bf16 pair (a in the low half), round to nearest even
// (one v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// sum over i < n of a[i] * b[i], one fmaf per term in index order (so the
// result does not depend on how the loads are grouped), with 16-byte loads
// when both rows are 16-byte aligned and n % 4 == 0
__device__ __forceinline__ float dot_f32(const float* a, const float* b, int n) {
  float s = 0.0f;
  if ((((uintptr_t)a | (uintptr_t)b) & 15u) == 0 && (n & 3) == 0) {
    const float4* a4 = (const float4*)a;
    const float4* b4 = (const float4*)b;
#pragma unroll 4
    for (int i = 0; i < (n >> 2); ++i) {
      const float4 x = a4[i], y = b4[i];
      s = fmaf(x.x, y.x, s);
      s = fmaf(x.y, y.y, s);
      s = fmaf(x.z, y.z, s);
      s = fmaf(x.w, y.w, s);
    }
  } else {
    for (int i = 0; i < n; ++i) s = fmaf(a[i], b[i], s);
  }
  return s;
}

// The ai-th expert (in id order) among those with rows, -1 past the last one.
// Blocks are numbered over the experts that have rows, so a step with few
// active experts launches few blocks and none waits only to find itself idle.
// Each wave computes it on its own (lane = expert, E <= kMaxExperts = 64).
__device__ __forceinline__ int active_expert(const int32_t* offsets, int gpe, int E, int ai) {
  const int lane = threadIdx.x & 63;
  bool has = false;
  if (lane < E) has = offsets[gpe * (lane + 1)] > offsets[gpe * lane];
  unsigned long long act = __ballot(has);
  if (ai >= __popcll(act)) return -1;
  for (int i = 0; i < ai; ++i) act &= act - 1ull;
  return __builtin_ctzll(act);
}

// g / (1 + e^-g) with the hardware reciprocal (about 1 ulp of fp32): every
// caller rounds the product with the up value to bf16, 2^14 times coarser
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// ---- launchers (each returns the launch status) -----------------------------

hipError_t launch_route_topk(const void* x, moe_dtype xdt, const void* w_router,
                             const float* b_router, int T, int d, int E, int k, float* logits,
                             int32_t* idx, float* gate, bool logits_given, hipStream_t s);

// Small batches (bf16, T <= 64, ceil(T/16) * ceil(E/16) <= 4): route, top-k
// and the permutation (counts, offsets, rows, LIS) in one workgroup.
bool route_permute_small_applies(moe_dtype xdt, int T, int E, int k);
// part_ws: route_part_bytes(...) bytes for the router GEMM split over d (NULL
// or 0 bytes: the workgroup computes the logits itself)
size_t route_part_bytes(moe_dtype xdt, int T, int d, int E, int k);
hipError_t launch_route_permute_small(const void* x, const void* w_router, const float* b_router,
                                      int T, int d, int E, int k, float* logits, int32_t* idx,
                                      float* gate, bool logits_given, int32_t* counts,
                                      int32_t* offsets, int32_t* row_assign, int32_t* assign_row,
                                      double* lis, float* part_ws, hipStream_t s);

size_t permute_ws_bytes(int T, int E, int k);
hipError_t launch_permute(const int32_t* idx, int T, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* row_assign, int32_t* assign_row,
                          double* lis, void* ws, hipStream_t s);

// Replica of expert `heavy` as slot E: its odd-ranked assignments move there;
// maps the E-slot permutation (counts, offsets, assign_row) to the E+1-slot one.
// Every output pointer may be NULL.
hipError_t launch_replica_remap(const int32_t* idx, const int32_t* counts, const int32_t* offsets,
                                const int32_t* assign_row, int T, int E, int k, int heavy,
                                int32_t* idx_out, int32_t* counts_out, int32_t* offsets_out,
                                int32_t* row_assign_out, int32_t* assign_row_out, double* lis_out,
                                hipStream_t s);

// Grouped expert FFN.  `mode` selects the projection: gate/up (SwiGLU or ReLU)
// producing H, or down producing gate-scaled fp32 rows.
struct FfnProblem {
  int T, d, F, E, k;
  moe_act act;
  moe_dtype dt;                  // activations and dense weights
  const void* x;                 // [T][d]
  const moe_experts* w;
  const int32_t* offsets;        // [E+1] or NULL (one expert, T rows)
  const int32_t* row_assign;     // row -> flat assignment, or NULL (identity, k = 1)
  const float* gate;             // gate per flat assignment, or NULL (1)
  float* y_rows;                 // [rows][d]
  void* H;                       // [rows][F] scratch (bf16 or fp32)
  int rows;                      // T * k
  int down_splits;               // K slices of the down pass (0 or 1: none); slice s
                                 // writes its partial sums to y_rows + s * rows * d
  float* y_direct;               // weight-streaming path only: if not NULL, the down
                                 // pass adds each gate-scaled row into y_direct[token]
                                 // [T][d] fp32 (zeroed by the caller) instead of
                                 // writing y_rows: the combine, fused
  bool rows_bf16;                // y_rows holds bf16 rows (tiled bf16 path only: see
                                 // ffn_rows_bf16_applies)
  const moe_experts* xw;         // if not NULL: expert xslot uses these bf16 weights
  int xslot;                     // ([N][K] per projection) instead of w's (tiled path)
  float* zero_y;                 // weight-streaming path: if not NULL, the gate/up grid
                                 // zeroes zero_y[0 .. T*d) first (the y that y_direct
                                 // accumulates into)
};
size_t ffn_ws_bytes(int rows, int F, moe_dtype dt);
// K slices for the down pass of a layer-sized problem: more, smaller tiles when
// one slice would leave the last round of tiles mostly idle; for INT4 weight
// streaming, K parts of the row-split down kernel.  A function of the shapes and
// of the weights' alignment (the workspace size depends on it).
int ffn_down_splits(int T, int d, int F, int E, int k, moe_dtype dt, const moe_experts* w);
hipError_t launch_grouped_ffn(const FfnProblem& p, hipStream_t s, hipEvent_t mid = nullptr);
// Whether the down pass can add its rows straight into y (FfnProblem::y_direct)
// with every y element receiving at most two of them: the weight-streaming
// path with k <= 2 (one K slice).  (The tiled pass with k = 1 could do the same
// with its two K slices; measured on the Switch-shaped layer, its fp32 atomics
// cost more than the combine launch they replace, so it keeps the combine.)
bool ffn_direct_applies(const FfnProblem& p);
// Whether the down pass can store its gate-scaled rows as bf16 (the 256x256
// tile path with dense bf16 experts)
bool ffn_rows_bf16_applies(const FfnProblem& p);

// Weight-streaming variant for few rows per expert (decode); same contract as
// launch_grouped_ffn.
bool stream_ffn_applies(const FfnProblem& p);
hipError_t launch_stream_ffn(const FfnProblem& p, hipStream_t s, hipEvent_t mid = nullptr);
// Row-split INT4 streaming kernel over K / parts of a K-long reduction with
// projections a and b (a == b for one projection), and the K parts its down
// pass takes for d_model d, d_ff F and E experts (1: the K-split kernel).
bool stream_rows_applies(int K, int parts, const moe_w4* a, const moe_w4* b);
int stream_down_parts(int d, int F, int E);
// INT4 projection w ([rows][K], decoded as documented for moe_w4) to bf16 out
// [rows][K], bit-identical to the weights the GEMM kernels decode in registers
hipError_t launch_dequant_int4(const moe_w4* w, int rows, int K, void* out, hipStream_t s);

// (expert, width) group of each assignment: 3 * idx + clamp(width, 2, 4) - 2.
hipError_t launch_mwq_group_ids(const int32_t* idx, const int32_t* widths, int n, int32_t* out,
                                hipStream_t s);

// Grouped FFN on nested 2/3/4-bit weights; rows grouped by (expert, width)
// (offsets [3E+1]).  Requires bf16 activations and d, F multiples of 512.
struct MwqProblem {
  int T, d, F, E, k;
  moe_act act;
  const void* x;                 // [T][d] bf16
  const moe_mwq_experts* w;
  const int32_t* offsets;        // [3E+1]
  const int32_t* row_assign;     // row -> flat assignment
  const float* gate;             // gate per flat assignment, or NULL (1)
  float* y_rows;                 // [rows][d]
  void* H;                       // [rows][F] bf16 scratch
  int rows;                      // T * k
};
// NULL if the shapes are supported, else the reason.
const char* mwq_ffn_unsupported(int T, int d, int F, int k);
hipError_t launch_mwq_ffn(const MwqProblem& p, hipStream_t s, hipEvent_t mid = nullptr);

// INT2 up projection of the contextual sparse down-projection: U [rows][F] fp32
// for every row of every expert (offsets [E+1]) and flags [E][F] = 1 where some
// row of the expert has |U| > thr[e].  Experts without rows leave their flags.
hipError_t launch_int2_up(const void* x, int T, int d, int F, int E, int k, const moe_wmwq* w,
                          const int32_t* offsets, const int32_t* row_assign, const float* thr,
                          float* U, uint8_t* flags, hipStream_t s);

// Contextual sparse down-projection (rows grouped by expert, offsets [E+1]).
struct FloeProblem {
  int T, d, F, E, k;
  const void* x;                 // [T][d] bf16
  const moe_floe_experts* w;
  const int32_t* offsets;        // [E+1]
  const int32_t* row_assign;     // row -> flat assignment
  const float* gate;             // gate per flat assignment, or NULL (1)
  float* U;                      // [rows][F] fp32 up outputs
  uint8_t* flags;                // [E][F]
  int32_t* list;                 // [E][F] kept channels of each expert, ascending
  int32_t* nnz;                  // [E]
  u16* Hc;                       // [rows][F] bf16 hidden values of the kept channels
  float* y_rows;                 // splits x [rows][d] gate-scaled partial sums
  int rows;
  int splits;
};
// Channel-list slices of the sparse down pass (pure function of the shapes).
int floe_down_splits(int d, int E);
const char* floe_unsupported(int T, int d, int F, int k);
hipError_t launch_floe_ffn(const FloeProblem& p, hipStream_t s, hipEvent_t mid = nullptr);

// Dense tiled GEMMs on the grouped-GEMM kernel (one group):
// Y[M][N] fp32 = A[M][K] . B[N][K]^T, K in ksplit slices (slice s adds nothing
// to the others: its partial sums go to Y + s * ystride); K % (128*ksplit) == 0.
hipError_t launch_gemm_bt(const u16* A, int lda, int M, const u16* B, int N, int K, float* Y,
                          int ksplit, size_t ystride, hipStream_t s);
// U = A . B^T [M][N]; H [M][N] bf16 = bf16(gates * silu(U)) at the cells whose
// bit is set in bits [M][N/32] and 0 elsewhere.  A kept cell's rank in its row
// (bitpre + popcount before it) indexes gates, kidx (its column) and ukept
// ([M][ksel] fp32 scratch for U).  K % 128 == 0, N % 32 == 0.
hipError_t launch_atomic_in(const u16* A, int M, const u16* B, int N, int K, const uint32_t* bits,
                            const int32_t* bitpre, const int32_t* kidx, const float* gates,
                            int ksel, float* ukept, u16* H, hipStream_t s);

// Atomic experts on an nr x nc router grid (atomic.hip).
// out = log_softmax over each row of the sum of nsplit partial [T][n] slices
hipError_t launch_log_softmax_rows(const float* l, int T, int n, float* out, hipStream_t s,
                                   int nsplit = 1, size_t split_stride = 0);
// exact top-K of fp32(pr[i] + pc[j]) per token (ties to the lower id i*nc + j),
// ids ascending, softmax gates, and the kept-cell bitmap with per-word prefixes
hipError_t launch_grid_topk(const float* pr, const float* pc, int T, int nr, int nc, int K,
                            int32_t* idx, float* gate, uint32_t* bits, int32_t* bitpre,
                            hipStream_t s);
size_t grid_permute_ws_bytes(int T, int N);
// expert-major permutation over N experts from the bitmap (token order inside
// an expert), counts, offsets, LIS
hipError_t launch_grid_permute(const uint32_t* bits, const int32_t* bitpre, int T, int N, int K,
                               int32_t* counts, int32_t* offsets, int32_t* row_assign,
                               int32_t* assign_row, double* lis, void* ws, hipStream_t s);
hipError_t launch_iota(int32_t* out, int n, hipStream_t s);

// Expert-centric execution of atomic experts (atomic_ec.hip).  Rows of expert
// n are offsets[n]..offsets[n+1]-1 (tokens ascending), row r is the kept pair
// a = row_assign[r] (token a / K, gate gates[a]).
// d a multiple of 512, at most 4096.
bool atomic_ec_supported(int d);
// expert ranges of the output side (partial sums [ranges][T][d] fp32)
int atomic_ec_ranges(int T, int d, int N);
// workspace: h [T*K] bf16 (256-byte aligned end), then the partial sums
size_t atomic_ec_ws_bytes(int T, int d, int N, int K);
// h[r] = bf16(gates[a] * silu(x[a / K] . w_in[n])) for every row r of every expert
hipError_t launch_atomic_ec_in(const u16* x, int T, int d, const u16* w_in, int N,
                               const int32_t* offsets, const int32_t* row_assign,
                               const float* gates, int K, u16* h, hipStream_t s);
// ypart[p][t] = sum over the experts n of range p, rows r of n with token t, of
// h[r] * w_out_rows[n]   (w_out_rows [N][d] bf16)
hipError_t launch_atomic_ec_out(const u16* h, const int32_t* offsets, const int32_t* row_assign,
                                int K, const u16* w_out_rows, int N, int d, int T, float* ypart,
                                hipStream_t s);
// y[t] = sum over ranges in order of ypart[p][t] (+ y_shared[t]), in ydt
hipError_t launch_atomic_ec_reduce(const float* ypart, int T, int d, int N,
                                   const float* y_shared, void* y, moe_dtype ydt, hipStream_t s);

// y[t] = sum over slots j, then over K slices s, of y_rows[s * split_stride +
// assign_row[t*k+j] * d], plus y_shared[t]; fixed order, so deterministic.
hipError_t launch_combine(const float* y_rows, const int32_t* assign_row, int T, int k, int d,
                          const float* y_shared, void* y, moe_dtype ydt, hipStream_t s,
                          int nsplit = 1, size_t split_stride = 0, bool rows_bf16 = false);

}  // namespace moe
