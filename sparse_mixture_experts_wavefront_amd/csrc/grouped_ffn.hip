// grouped_ffn.hip -- grouped expert FFN over expert-major rows.
//
// "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale" -- What
// carries the argument and Figure 3: rows of each active expert are contiguous,
// so each expert is one dense GEMM and the whole layer one grouped GEMM.
// "FloE: On-the-Fly MoE Inference on Memory-constrained GPU" -- What carries the
// argument, Core claim, Figure 11: an expert is W_gate, W_up, W_down; SiLU acts
// on the gate projection, the up projection multiplies it, and that product is
// the input of the down projection.
// "D^2MoE: Dual Routing and Dynamic Scheduling for Efficient On-Device MoE-based
// LLM Serving" -- What carries the argument (asymmetric quantisation), the
// free-parameter ledger (group size 128) and Figure 8 (dequantisation inside
// the GEMM): INT4 weights are decoded while they are staged, never stored
// decoded in HBM.
//
// Two passes per expert group, each a tiled bf16 MFMA GEMM (fp32 accumulate):
//   gate/up : H[r] = act(x[token(r)] W_gate^T, x[token(r)] W_up^T)  -> bf16
//   down    : y_rows[r] = gate(r) * H[r] W_down^T                    -> fp32
// The tile map is ragged and lives on the device: every block reads offsets[],
// forms the per-expert tile prefix with one wave scan, and finds its own
// (expert, row tile); blocks past the last tile exit.  Block ids are remapped
// so that consecutive ids on one XCD (ids that differ by 8) take the row tiles
// of one weight panel, which then stays in that XCD's L2.
// Tile: BM x BN x 64, 256 threads as 2x2 waves, 32x32x16 MFMA.  Operands are
// K-contiguous in both A and B; LDS rows are 64 bf16 with 16-byte chunks
// XOR-swizzled by (row & 7) so MFMA fragment reads do not collide on banks.
// Global->LDS staging is double buffered: the loads of tile k+1 are in flight
// while the MFMAs of tile k run.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBK = 64;
constexpr int kThreads = 256;

enum Mode { kGateUpSwiglu = 0, kUpRelu = 1, kDown = 2 };

struct TileArgs {
  const u16* A;            // gate/up: x [T][lda]; down: H [rows][lda]
  int lda;
  const int32_t* gather;   // gate/up: row -> flat assignment (token = a / k); NULL identity
  int k;
  const u16* B0;           // dense bf16 weights [E][N][K] (gate or W_in or down)
  const u16* B1;           // up weights for SwiGLU
  const int32_t* q0;       // INT4 words [E][N][K/8] (NULL: dense)
  const int32_t* q1;
  const u16* s0;           // fp16 scales [E][N][K/128]
  const u16* s1;
  const u16* z0;           // fp16 zero points [E][N][K/128]
  const u16* z1;
  int N, K;
  const int32_t* offsets;  // [E+1] or NULL
  int E, rows;
  u16* H;                  // gate/up output [rows][N]
  float* Y;                // down output [rows][N]
  const int32_t* gate_map; // down: row -> flat assignment for the gate; NULL: gate index = row
  const float* gate;       // gate per flat assignment; NULL: 1
  int m_tiles_max, n_tiles;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

__device__ __forceinline__ float fp16_to_f32(u16 h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Decode 8 INT4 weights (one int32 word, low nibble first) to bf16 with
// W = bf16_RNE( fp32( fp32(q) - z ) * s ), each fp32 op rounded separately.
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float s, float z) {
  u32x4 out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float q0 = (float)((w >> (8 * p)) & 0xfu);
    const float q1 = (float)((w >> (8 * p + 4)) & 0xfu);
    const float a0 = __fsub_rn(q0, z), a1 = __fsub_rn(q1, z);
    const float b0 = __fmul_rn(a0, s), b1 = __fmul_rn(a1, s);
    out[p] = (uint32_t)f32_to_bf16(b0) | ((uint32_t)f32_to_bf16(b1) << 16);
  }
  return out;
}

template <int BM, int BN, int MODE, bool INT4>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(TileArgs p) {
  constexpr int NMAT = (MODE == kGateUpSwiglu) ? 2 : 1;
  constexpr int WM = BM / 2, WN = BN / 2;      // wave tile
  constexpr int MI = WM / 32, NI = WN / 32;    // 32x32 MFMA blocks per wave
  constexpr int AJ = BM / 32, BJ = BN / 32;    // 16-byte chunks per thread per stage
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");

  extern __shared__ __align__(16) u16 smem[];
  u16* As = smem;                              // [2][BM*64]
  u16* Bs = smem + 2 * BM * kBK;               // [2][NMAT][BN*64]
  __shared__ int s_tile[3];                    // expert, first row, valid rows

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // ---- ragged tile map (device side) ----
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int v = (bid & 7) * (nb >> 3) + (bid >> 3);   // XCD-contiguous virtual id
  const int n_tile = v / p.m_tiles_max;
  const int m_tile = v - n_tile * p.m_tiles_max;
  if (n_tile >= p.n_tiles) return;
  if (wid == 0) {
    int cnt = 0, first = 0;
    if (p.offsets) {
      if (lane < p.E) {
        first = p.offsets[lane];
        cnt = p.offsets[lane + 1] - first;
      }
    } else if (lane == 0) {
      cnt = p.rows;
    }
    const int tiles = (cnt + BM - 1) / BM;
    int incl = tiles;
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const int excl = incl - tiles;
    if (lane == 0) s_tile[0] = -1;
    // (one lane matches; a wave executes its LDS writes in program order)
    if (m_tile >= excl && m_tile < incl) {
      s_tile[0] = lane;
      s_tile[1] = first + (m_tile - excl) * BM;
      s_tile[2] = min(BM, cnt - (m_tile - excl) * BM);
    }
  }
  __syncthreads();
  const int expert = s_tile[0];
  if (expert < 0) return;
  const int row0 = s_tile[1], rvalid = s_tile[2];
  const int n0 = n_tile * BN;

  // ---- per-thread global pointers ----
  const int kc = tid & 7;               // this thread's 16-byte chunk inside a 64-wide K slice
  const u16* a_ptr[AJ];
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    const int r = (tid >> 3) + 32 * j;
    const int gr = row0 + min(r, rvalid - 1);
    const int src = p.gather ? (p.gather[gr] / p.k) : gr;
    a_ptr[j] = p.A + (size_t)src * p.lda + kc * 8;
  }
  const size_t wstride = (size_t)p.N * p.K;
  const u16* b_ptr[NMAT][BJ];
  const int32_t* q_ptr[NMAT][BJ];
  const u16* sz_ptr[NMAT][BJ][2];
  const int kq = p.K >> 3;        // int32 words per INT4 row
  const int kg = p.K >> 7;        // groups per INT4 row
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      const int n = min(n0 + (tid >> 3) + 32 * j, p.N - 1);
      if constexpr (!INT4) {
        const u16* B = m ? p.B1 : p.B0;
        b_ptr[m][j] = B + (size_t)expert * wstride + (size_t)n * p.K + kc * 8;
      } else {
        const int32_t* Q = m ? p.q1 : p.q0;
        q_ptr[m][j] = Q + ((size_t)expert * p.N + n) * kq + kc;
        sz_ptr[m][j][0] = (m ? p.s1 : p.s0) + ((size_t)expert * p.N + n) * kg;
        sz_ptr[m][j][1] = (m ? p.z1 : p.z0) + ((size_t)expert * p.N + n) * kg;
      }
    }

  u32x4 ra[AJ];
  u32x4 rb[NMAT][BJ];
  const int nk = (p.K + kBK - 1) / kBK;

  auto load_stage = [&](int kt) {
    const int k0 = kt * kBK;
    const bool kin = (k0 + kc * 8) < p.K;
#pragma unroll
    for (int j = 0; j < AJ; ++j)
      ra[j] = kin ? *(const u32x4*)(a_ptr[j] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        if constexpr (!INT4) {
          rb[m][j] = kin ? *(const u32x4*)(b_ptr[m][j] + k0) : u32x4{0, 0, 0, 0};
        } else {
          if (kin) {
            const uint32_t w = (uint32_t)q_ptr[m][j][k0 >> 3];
            const int g = k0 >> 7;
            const float s = fp16_to_f32(sz_ptr[m][j][0][g]);
            const float z = fp16_to_f32(sz_ptr[m][j][1][g]);
            rb[m][j] = dequant8(w, s, z);
          } else {
            rb[m][j] = u32x4{0, 0, 0, 0};
          }
        }
      }
  };
  auto store_stage = [&](int buf) {
    u16* as = As + buf * BM * kBK;
#pragma unroll
    for (int j = 0; j < AJ; ++j) *(u32x4*)(as + swz((tid >> 3) + 32 * j, kc)) = ra[j];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      u16* bs = Bs + (buf * NMAT + m) * BN * kBK;
#pragma unroll
      for (int j = 0; j < BJ; ++j) *(u32x4*)(bs + swz((tid >> 3) + 32 * j, kc)) = rb[m][j];
    }
  };

  f32x16 acc[NMAT][MI][NI];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.0f;

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int fr = lane & 31, fk = lane >> 5;   // fragment row and K half
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
    const u16* as = As + cur * BM * kBK;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int chunk = kk * 2 + fk;
      bf16x8 af[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[i] = as_bf16x8(*(const u32x4*)(as + swz(wm * WM + i * 32 + fr, chunk)));
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const u16* bs = Bs + (cur * NMAT + m) * BN * kBK;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const bf16x8 bfr = as_bf16x8(*(const u32x4*)(bs + swz(wn * WN + j * 32 + fr, chunk)));
#pragma unroll
          for (int i = 0; i < MI; ++i) acc[m][i][j] = mfma32(af[i], bfr, acc[m][i][j]);
        }
      }
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue; 32x32 C layout: reg r -> row 8*(r/4) + 4*(lane/32) + r%4, col lane%32 ----
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
      if (row >= rvalid) continue;
      const int grow = row0 + row;
      float gscale = 1.0f;
      if constexpr (MODE == kDown) {
        if (p.gate) gscale = p.gate[p.gate_map ? p.gate_map[grow] : grow];
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int col = n0 + wn * WN + j * 32 + fr;
        if (col >= p.N) continue;
        if constexpr (MODE == kGateUpSwiglu) {
          const float g = acc[0][i][j][r], u = acc[1][i][j][r];
          p.H[(size_t)grow * p.N + col] = f32_to_bf16(silu_f32(g) * u);
        } else if constexpr (MODE == kUpRelu) {
          p.H[(size_t)grow * p.N + col] = f32_to_bf16(fmaxf(acc[0][i][j][r], 0.0f));
        } else {
          p.Y[(size_t)grow * p.N + col] = gscale * acc[0][i][j][r];
        }
      }
    }
}

// ---- fp32 layers: plain per-output dot products (no fp32 MFMA needed at these sizes) ----

__global__ __launch_bounds__(256) void ffn_f32_up_kernel(const float* __restrict__ x, int d,
                                                         const float* __restrict__ wg,
                                                         const float* __restrict__ wu, int F,
                                                         const int32_t* __restrict__ offsets,
                                                         int E, const int32_t* __restrict__ gather,
                                                         int k, int rows, int relu,
                                                         float* __restrict__ H) {
  const long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (long long)rows * F) return;
  const int r = (int)(id / F), f = (int)(id % F);
  int e = 0;
  if (offsets)
    while (e + 1 < E && offsets[e + 1] <= r) ++e;
  const int t = gather ? gather[r] / k : r;
  const float* xr = x + (size_t)t * d;
  const float* wur = wu + ((size_t)e * F + f) * d;
  float u = 0.0f;
  for (int i = 0; i < d; ++i) u = fmaf(xr[i], wur[i], u);
  float h;
  if (relu) {
    h = fmaxf(u, 0.0f);
  } else {
    const float* wgr = wg + ((size_t)e * F + f) * d;
    float g = 0.0f;
    for (int i = 0; i < d; ++i) g = fmaf(xr[i], wgr[i], g);
    h = (g / (1.0f + expf(-g))) * u;
  }
  H[(size_t)r * F + f] = h;
}

__global__ __launch_bounds__(256) void ffn_f32_down_kernel(const float* __restrict__ H, int F,
                                                           const float* __restrict__ wd, int d,
                                                           const int32_t* __restrict__ offsets,
                                                           int E, const int32_t* __restrict__ gmap,
                                                           const float* __restrict__ gate,
                                                           int rows, float* __restrict__ Y) {
  const long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (long long)rows * d) return;
  const int r = (int)(id / d), i = (int)(id % d);
  int e = 0;
  if (offsets)
    while (e + 1 < E && offsets[e + 1] <= r) ++e;
  const float* hr = H + (size_t)r * F;
  const float* wr = wd + ((size_t)e * d + i) * F;
  float s = 0.0f;
  for (int f = 0; f < F; ++f) s = fmaf(hr[f], wr[f], s);
  const float g = gate ? gate[gmap ? gmap[r] : r] : 1.0f;
  Y[(size_t)r * d + i] = g * s;
}

template <int BM, int BN, int MODE, bool INT4>
hipError_t run_tiles(TileArgs a, hipStream_t s) {
  constexpr int NMAT = (MODE == kGateUpSwiglu) ? 2 : 1;
  const int m_tiles_max = (a.rows + BM - 1) / BM + min(a.E, a.rows);
  a.m_tiles_max = m_tiles_max;
  a.n_tiles = (a.N + BN - 1) / BN;
  long long nblk = (long long)m_tiles_max * a.n_tiles;
  nblk = (nblk + 7) / 8 * 8;
  const size_t lds = (size_t)2 * (BM + NMAT * BN) * kBK * sizeof(u16);
  auto kern = grouped_gemm_kernel<BM, BN, MODE, INT4>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

size_t ffn_ws_bytes(int rows, int F, moe_dtype dt) {
  return (size_t)rows * F * (dt == MOE_DT_F32 ? 4 : 2);
}

hipError_t launch_grouped_ffn(const FfnProblem& p, hipStream_t s, hipEvent_t mid) {
  if (p.rows == 0) return hipSuccess;
  const bool relu = p.act == MOE_ACT_RELU;
  const int E = p.offsets ? p.E : 1;
  if (p.dt == MOE_DT_F32) {
    const float* wg = (const float*)p.w->w_gate;
    const float* wu = (const float*)p.w->w_up;
    const float* wd = (const float*)p.w->w_down;
    const long long n1 = (long long)p.rows * p.F, n2 = (long long)p.rows * p.d;
    hipLaunchKernelGGL(ffn_f32_up_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s,
                       (const float*)p.x, p.d, wg, wu, p.F, p.offsets, E, p.row_assign, p.k,
                       p.rows, relu ? 1 : 0, (float*)p.H);
    if (mid) (void)hipEventRecord(mid, s);
    hipLaunchKernelGGL(ffn_f32_down_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s,
                       (const float*)p.H, p.F, wd, p.d, p.offsets, E, p.row_assign, p.gate,
                       p.rows, p.y_rows);
    return hipGetLastError();
  }
  const bool int4 = p.w->q_up != nullptr;
  TileArgs a = {};
  a.k = p.k;
  a.offsets = p.offsets;
  a.E = E;
  a.rows = p.rows;
  // pass 1: gate/up
  a.A = (const u16*)p.x;
  a.lda = p.d;
  a.gather = p.row_assign;
  a.N = p.F;
  a.K = p.d;
  a.H = (u16*)p.H;
  if (int4) {
    const moe_w4* qg = p.w->q_gate;
    const moe_w4* qu = p.w->q_up;
    if (relu) {
      a.q0 = qu->q; a.s0 = qu->scale; a.z0 = qu->zero;
    } else {
      a.q0 = qg->q; a.s0 = qg->scale; a.z0 = qg->zero;
      a.q1 = qu->q; a.s1 = qu->scale; a.z1 = qu->zero;
    }
  } else {
    a.B0 = (const u16*)(relu ? p.w->w_up : p.w->w_gate);
    a.B1 = (const u16*)p.w->w_up;
  }
  hipError_t e;
  if (relu)
    e = int4 ? run_tiles<128, 128, kUpRelu, true>(a, s) : run_tiles<128, 128, kUpRelu, false>(a, s);
  else
    e = int4 ? run_tiles<128, 128, kGateUpSwiglu, true>(a, s)
             : run_tiles<128, 128, kGateUpSwiglu, false>(a, s);
  if (e != hipSuccess) return e;
  if (mid) {
    e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
  }
  // pass 2: down
  TileArgs b = {};
  b.k = p.k;
  b.offsets = p.offsets;
  b.E = E;
  b.rows = p.rows;
  b.A = (const u16*)p.H;
  b.lda = p.F;
  b.gather = nullptr;
  b.N = p.d;
  b.K = p.F;
  b.Y = p.y_rows;
  b.gate_map = p.row_assign;
  b.gate = p.gate;
  if (int4) {
    b.q0 = p.w->q_down->q; b.s0 = p.w->q_down->scale; b.z0 = p.w->q_down->zero;
    return run_tiles<128, 128, kDown, true>(b, s);
  }
  b.B0 = (const u16*)p.w->w_down;
  return run_tiles<128, 128, kDown, false>(b, s);
}

}  // namespace moe
