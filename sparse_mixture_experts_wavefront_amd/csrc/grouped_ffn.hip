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
// so that each XCD (block id % 8) takes a contiguous share of the tiles, whose
// row tiles of one weight panel then meet in that XCD's L2.
// Two tiled kernels: the 256x256x64 DMA-staged kernel (bf16, K % 128 == 0: the
// layer path) and a 128x128x64 register-staged kernel (INT4 weights decoded
// while staged, and any other shape).
#include <mutex>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kAttrDevices = 64;  // devices whose kernel attributes are cached

// kAtomIn: one matrix (the input side of the atomic experts); at the cells a
// per-row bitmap keeps the output is bf16(gate * silu(acc)), elsewhere 0.  The
// kept cells' fp32 values are listed in LDS (or, for a dense tile, in a compact
// [rows][ksel] array at the cell's rank in its row, where the gates and ids of
// the row also sit).
enum Mode { kGateUpSwiglu = 0, kUpRelu = 1, kDown = 2, kAtomIn = 3 };
// kAtomIn: kept cells of a tile listed in LDS (the operand buffer holds 8192
// entries; the last 64 take the writes of lanes whose cell is not kept)
constexpr int kAtomTileCap = 8192 - 64;

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
  int ksplit;              // K slices (down only): slice s covers K [s*K/ksplit, +K/ksplit)
  size_t ystride;          // elements between the partial outputs of two slices
  int ybf16;               // down (256x256 path): Y holds bf16 rows (RNE), not fp32
  const u16* xB0;          // if not NULL, expert xslot takes its weights from xB0 (and
  const u16* xB1;          // xB1, up for SwiGLU), [N][K] each, instead of B0/B1 (256x256 path)
  int xslot;
  const uint32_t* bits;    // kAtomIn: [rows][wpr] kept cells, bit c%32 of word c/32
  const int32_t* bitpre;   // kAtomIn: [rows][wpr] kept cells of the row before the word
  int wpr;                 // kAtomIn: words per row (N / 32)
  int ksel;                // kAtomIn: kept cells per row
  float* ukept;            // kAtomIn: [rows][ksel] fp32 values of the kept cells
  const int32_t* kidx;     // kAtomIn: [rows][ksel] column of each kept cell (ascending)
};

// LDS rows of 64 bf16 (128 B).  The LDS has 64 banks of 4 bytes and serves a
// 16-byte-per-lane read 16 lanes per pass (256 B); the 16 rows one pass reads
// land on distinct 16-byte bank groups when chunk c of row r is stored at
// position c ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3); }

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
  // down: the gate of tile row tid, loaded now (its latency passes under the
  // main loop) and staged in LDS for the epilogue
  float gpre = 1.0f;
  if constexpr (MODE == kDown) {
    if (p.gate && tid < BM) {
      const int gr = row0 + min(tid, rvalid - 1);
      gpre = p.gate[p.gate_map ? p.gate_map[gr] : gr];
    }
  }

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
  // INT4: the stage's raw word, scale and zero point; decoded in store_stage,
  // after the current stage's MFMAs, so the loads of the next stage are in
  // flight under them rather than waited for at once
  uint32_t rq[INT4 ? NMAT : 1][INT4 ? BJ : 1];
  u16 rs[INT4 ? NMAT : 1][INT4 ? BJ : 1], rz[INT4 ? NMAT : 1][INT4 ? BJ : 1];
  bool rkin = false;
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
          // past K: the stage's first word and group (in bounds), decoded to zeros
          const int kq = kin ? k0 : 0;
          rq[m][j] = (uint32_t)q_ptr[m][j][kq >> 3];
          rs[m][j] = sz_ptr[m][j][0][kq >> 7];
          rz[m][j] = sz_ptr[m][j][1][kq >> 7];
        }
      }
    rkin = kin;
  };
  auto store_stage = [&](int buf) {
    u16* as = As + buf * BM * kBK;
#pragma unroll
    for (int j = 0; j < AJ; ++j) *(u32x4*)(as + swz((tid >> 3) + 32 * j, kc)) = ra[j];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      u16* bs = Bs + (buf * NMAT + m) * BN * kBK;
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        if constexpr (INT4)
          rb[m][j] = rkin ? dequant8(rq[m][j], fp16_to_f32(rs[m][j]), fp16_to_f32(rz[m][j]))
                          : u32x4{0, 0, 0, 0};
        *(u32x4*)(bs + swz((tid >> 3) + 32 * j, kc)) = rb[m][j];
      }
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
  float* gsc = (float*)smem;  // the operand buffers are free (barrier above)
  if constexpr (MODE == kDown) {
    if (tid < BM) gsc[tid] = gpre;
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
      if (row >= rvalid) continue;
      const int grow = row0 + row;
      float gscale = 1.0f;
      if constexpr (MODE == kDown) gscale = gsc[row];
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

// ---- shared pieces of the 256x256 tiled kernel ---------------------------------------
constexpr int kV2BM = 256, kV2GroupM = 8;  // tile rows; row tiles per column-strip group
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void dma16(const void* g, u16* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}
// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14])
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int v3_pos(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
__device__ __forceinline__ int v3_off(int row, int chunk) { return row * 64 + (v3_pos(row, chunk) << 3); }

// ---- tiled grouped GEMM for many rows per expert: 256x256x64 tiles -------------------
//
// 256 threads as 2x2 waves, each owning a 128x128 quarter of the output tile with
// 32x32x16 bf16 MFMAs (16 fp32x16 accumulators, 256 registers per lane).  A and B
// stage through two 64 KB LDS buffers with global_load_lds_dwordx4 (each lane's
// 16 bytes land at base + 16*lane: no registers hold tiles in flight); each
// stage covers 64 K values, so every row contributes one full 128-byte line.
// LDS rows are 128 bytes; chunk c of row r sits at position c ^ ((r >> 1) & 7),
// which puts the 16 rows one 256-byte LDS pass serves on 16 distinct bank
// groups (the LDS has 64 banks of 4 bytes and serves 16-byte reads 16 lanes per
// pass).  Measured on MI355X: LDS reads reach ~80 B/clk/CU from 4 waves and bf16
// MFMA ~1.95 PFLOP/s, so the schedule is built around the LDS: every MFMA is
// followed by at most one other memory instruction, fragment reads run two K
// quarters ahead (four register sets), and one barrier per stage, after its
// second quarter, publishes the next stage and frees the current buffer for the
// DMA of the stage two ahead, issued during the third and fourth quarters.
// Real tiles are numbered expert by expert, in groups of up to 8 of the
// expert's row tiles per column strip, and each XCD takes a contiguous eighth
// of them, so its concurrent tiles share A and B slices in its L2.  The down pass may split K into slices (partial rows
// reduced by the combine).  Epilogues avoid per-element waits: the SwiGLU and
// ReLU modes feed the MFMA weights-first, so each lane ends with four
// consecutive output columns per register quad; their tiles are assembled in
// the free LDS with 8-byte writes and leave in 16-byte buffer stores; the down
// rows take their gates from LDS (loaded before the main loop) and leave
// through a bounds-checked buffer resource.
template <int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_tile_kernel(TileArgs p) {
  constexpr int BM = 256, BK = 64;
  constexpr int STAGE = BM * BK;
  __shared__ __align__(16) u16 sA0[STAGE], sA1[STAGE];
  __shared__ __align__(16) u16 sB0[STAGE], sB1[STAGE];
  __shared__ int s_tile[5];  // expert, first row, valid rows, column tile, K slice

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // Tile map.  Wave 0 scans the experts' row-tile counts; the real tiles are
  // numbered K slice first (slice ks covers K [ks*K/ksplit, +K/ksplit) and
  // writes its partial sums to Y + ks*ystride, which the combine adds), then
  // expert by expert, and inside an expert in groups of up to kV2GroupM of its
  // row tiles per column strip (a group never mixes experts, so its tiles share
  // one weight strip).  Block bid runs on XCD bid % 8 and takes tile
  // (bid % 8) * ceil(R/8) + bid / 8 of the R real tiles: every XCD gets a
  // contiguous eighth of the real tiles (equal work, and neighbouring tiles
  // share A and B slices in that XCD's L2); blocks past them exit at once.
  if (wid == 0) {
    // up to 128 experts: lane holds experts lane and lane + 64 (the second only
    // when a replica slot makes E = 65)
    int cnt[2] = {0, 0}, first[2] = {0, 0}, tiles[2], excl[2];
    if (p.offsets) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ex = lane + 64 * c;
        if (ex < p.E) {
          first[c] = p.offsets[ex];
          cnt[c] = p.offsets[ex + 1] - first[c];
        }
      }
    } else if (lane == 0) {
      cnt[0] = p.rows;
    }
    int m_real = 0;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      tiles[c] = (cnt[c] + BM - 1) / BM;
      int incl = tiles[c];
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      excl[c] = m_real + incl - tiles[c];
      m_real += __shfl(incl, 63, 64);
    }
    const int slice_tiles = m_real * p.n_tiles;
    const int total = slice_tiles * p.ksplit;
    const int per_xcd = (total + 7) >> 3;
    const int loc = blockIdx.x >> 3;
    int t = (blockIdx.x & 7) * per_xcd + loc;
    if (lane == 0) s_tile[0] = -1;
    if (loc < per_xcd && t < total) {
      const int ksl = t / slice_tiles;
      t -= ksl * slice_tiles;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int u = t - excl[c] * p.n_tiles;  // tile index inside expert lane + 64c
        if (u >= 0 && u < tiles[c] * p.n_tiles) {  // exactly one (lane, c)
          const int per_group = kV2GroupM * p.n_tiles;
          const int g = u / per_group;
          const int first_m = g * kV2GroupM;
          const int gm = min(tiles[c] - first_m, kV2GroupM);
          const int in_g = u - g * per_group;
          const int m_loc = first_m + in_g % gm;
          s_tile[0] = lane + 64 * c;
          s_tile[1] = first[c] + m_loc * BM;
          s_tile[2] = min(BM, cnt[c] - m_loc * BM);
          s_tile[3] = in_g / gm;
          s_tile[4] = ksl;
        }
      }
    }
  }
  __syncthreads();
  const int expert = __builtin_amdgcn_readfirstlane(s_tile[0]);
  if (expert < 0) return;
  const int row0 = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int rvalid = __builtin_amdgcn_readfirstlane(s_tile[2]);
  const int n_tile = __builtin_amdgcn_readfirstlane(s_tile[3]);
  const int ks = __builtin_amdgcn_readfirstlane(s_tile[4]);
  const int kslice = p.K / p.ksplit;
  // down: the gate of this thread's row of the tile, loaded now so that its
  // latency passes under the main loop (staged in LDS for the epilogue)
  float gpre = 1.0f;
  if constexpr (MODE == kDown) {
    if (p.gate) {
      const int gr = row0 + min(tid, rvalid - 1);
      gpre = p.gate[p.gate_map ? p.gate_map[gr] : gr];
    }
  }

  // DMA: instruction j (0..7 A, 8..15 B) of wave w fills LDS rows (w*8+j%8)*8 ..
  // +8 (1 KB); lane L feeds row (w*8+j%8)*8 + L/8 at 16-byte position L%8.  The
  // first two stages issue their B (weight) instructions before the A ones,
  // whose addresses may wait for the gather map.
  const u16* src[16];
  const size_t wstride = (size_t)p.N * p.K;
  // source rows of the 8 A rows this lane feeds; with a gather map, its 8
  // entries are loaded together (one memory round trip, not eight)
  int srow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) srow[j] = row0 + min((wid * 8 + j) * 8 + (lane >> 3), rvalid - 1);
  if (p.gather) {
    int gv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) gv[j] = p.gather[srow[j]];
#pragma unroll
    for (int j = 0; j < 8; ++j) srow[j] = gv[j] / p.k;
  }
  // the extra slot (a replica's decoded weights) reads its own [N][K] matrices
  const bool xs = p.xB0 != nullptr && expert == p.xslot;
  const u16* B0 = xs ? p.xB0 : p.B0 + (size_t)expert * wstride;
  const u16* B1 = MODE != kGateUpSwiglu ? nullptr : xs ? p.xB1 : p.B1 + (size_t)expert * wstride;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (wid * 8 + j) * 8 + (lane >> 3);
    const int c = v3_pos(r, lane & 7);
    src[j] = p.A + (size_t)srow[j] * p.lda + c * 8;
    const u16* Bm;
    int n;
    if constexpr (MODE == kGateUpSwiglu) {
      Bm = (r < 128) ? B0 : B1;
      n = n_tile * 128 + (r & 127);
    } else {
      Bm = B0;
      n = n_tile * 256 + r;
    }
    n = min(n, p.N - 1);
    src[8 + j] = Bm + (size_t)n * p.K + c * 8;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) src[j] += (size_t)ks * kslice;
  const int nk = kslice / BK;
  const int wbase = __builtin_amdgcn_readfirstlane(wid) * 8 * 512;
  auto dma = [&](u16* sa, u16* sb, int kt, int j) {
    const int k0 = min(kt, nk - 1) * BK;  // past the end: reload the last slice (never read)
    dma16(src[j] + k0, (j < 8 ? sa : sb) + wbase + (j & 7) * 512);
  };

  const int fr = lane & 31, fk = lane >> 5;
  if constexpr (MODE != kAtomIn) {
    if (rvalid <= 128) {
      // ---- half tile: at most 128 valid rows (an expert's remainder).  All four
      // waves take rows 0..127 and wave w a quarter of the columns (gate/up: the
      // gate and up columns w*32..+32 of the strip), so each wave runs 8 MFMAs
      // per K quarter instead of 16 and the tile costs about half a full one.
      // Staging, swizzle and pipeline are those of the full tile below.
      f32x16 hacc[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) hacc[i][j][r] = 0.0f;
      const int wq = __builtin_amdgcn_readfirstlane(wid);
      auto hbrow = [&](int j) {
        if constexpr (MODE == kGateUpSwiglu) return j == 0 ? wq * 32 : 128 + wq * 32;
        else return wq * 64 + j * 32;
      };
      // fragment f (0..3 A rows f*32.., 4..5 B columns) of K quarter kk
      auto hread = [&](const u16* sa, const u16* sb, int kk, int f, bf16x8 (&af)[4],
                       bf16x8 (&bfr)[4]) {
        const int c = kk * 2 + fk;
        if (f < 4)
          af[f] = as_bf16x8(*(const u32x4*)(sa + v3_off(f * 32 + fr, c)));
        else
          bfr[f - 4] = as_bf16x8(*(const u32x4*)(sb + v3_off(hbrow(f - 4) + fr, c)));
      };
      constexpr int kReadH[6] = {0, 4, 5, 1, 2, 3};
      bf16x8 ha[4][4], hb[4][4];  // [quarter set][fragment]
      auto hquarter = [&](int q, const u16* sa_r, const u16* sb_r, int kk_r, int r, u16* sa_d,
                          u16* sb_d, int kt_dma, int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          hacc[m >> 1][m & 1] = mfma32(ha[q][m >> 1], hb[q][m & 1], hacc[m >> 1][m & 1]);
          if (m < 6) hread(sa_r, sb_r, kk_r, kReadH[m], ha[r], hb[r]);
          if (j0 >= 0) dma(sa_d, sb_d, kt_dma, j0 + m);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      auto hstage = [&](u16* sa, u16* sb, u16* na, u16* nb_, int kt) __attribute__((always_inline)) {
        hquarter(0, sa, sb, 2, 2, sa, sb, 0, -1);
        hquarter(1, sa, sb, 3, 3, sa, sb, 0, -1);
        wait_vm_lgkm0<0>();
        block_barrier();
        hquarter(2, na, nb_, 0, 0, sa, sb, kt + 2, 0);
        hquarter(3, na, nb_, 1, 1, sa, sb, kt + 2, 8);
      };
#pragma unroll
      for (int j = 8; j < 16; ++j) dma(sA0, sB0, 0, j);
#pragma unroll
      for (int j = 8; j < 16; ++j) dma(sA1, sB1, 1, j);
#pragma unroll
      for (int j = 0; j < 8; ++j) dma(sA0, sB0, 0, j);
#pragma unroll
      for (int j = 0; j < 8; ++j) dma(sA1, sB1, 1, j);
      wait_vm_lgkm0<8>();
      block_barrier();
#pragma unroll
      for (int f = 0; f < 6; ++f) hread(sA0, sB0, 0, kReadH[f], ha[0], hb[0]);
#pragma unroll
      for (int f = 0; f < 6; ++f) hread(sA0, sB0, 1, kReadH[f], ha[1], hb[1]);
      for (int kt = 0; kt < nk; kt += 2) {
        hstage(sA0, sB0, sA1, sB1, kt);
        hstage(sA1, sB1, sA0, sB0, kt + 1);
      }
      wait_vm_lgkm0<0>();
      __syncthreads();  // every wave is done with the operand buffers
      // output element (i, j, r): tile row i*32 + 8*(r/4) + 4*fk + r%4
      if constexpr (MODE == kGateUpSwiglu) {
        auto hp = [&](int row, int col) -> u16* {
          return sA0 + row * 128 + (((col >> 3) ^ (row & 7)) << 3) + (col & 7);
        };
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
            *hp(row, wq * 32 + fr) = f32_to_bf16(silu_f32(hacc[i][0][r]) * hacc[i][1][r]);
          }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int l = q * 256 + tid;
          const int row = l >> 4, c = l & 15;
          const int col = n_tile * 128 + c * 8;
          if (row < rvalid && col < p.N)
            *(u32x4*)(p.H + (size_t)(row0 + row) * p.N + col) = *(const u32x4*)hp(row, c * 8);
        }
      } else if constexpr (MODE == kUpRelu) {
        auto hp = [&](int row, int col) -> u16* {
          return (row < 64 ? sA0 : sA1) + (row & 63) * 256 + (((col >> 3) ^ (row & 7)) << 3) +
                 (col & 7);
        };
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
#pragma unroll
            for (int j = 0; j < 2; ++j)
              *hp(row, wq * 64 + j * 32 + fr) = f32_to_bf16(fmaxf(hacc[i][j][r], 0.0f));
          }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int l = q * 256 + tid;
          const int row = l >> 5, c = l & 31;
          const int col = n_tile * 256 + c * 8;
          if (row < rvalid && col < p.N)
            *(u32x4*)(p.H + (size_t)(row0 + row) * p.N + col) = *(const u32x4*)hp(row, c * 8);
        }
      } else {  // kDown
        float* gsc = (float*)sA0;
        gsc[tid] = gpre;
        __syncthreads();
        const int esz = p.ybf16 ? 2 : 4;  // bytes per output element
        const __amdgpu_buffer_rsrc_t yres = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const char*)p.Y + ((size_t)ks * p.ystride + (size_t)row0 * p.N) * esz),
            (short)0, rvalid * p.N * esz, 0x00020000);
        const int wcol0 = n_tile * 256 + wq * 64;
        auto rows = [&](auto whole, auto bf16) __attribute__((always_inline)) {
          constexpr bool WHOLE = decltype(whole)::value;  // the wave's 64 columns all < N
          constexpr bool BF = decltype(bf16)::value;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = i * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
              const float g = gsc[row];
              const int off = (row * p.N + wcol0 + fr) * (BF ? 2 : 4);
#pragma unroll
              for (int j = 0; j < 2; ++j)
                if (WHOLE || wcol0 + j * 32 + fr < p.N) {
                  if constexpr (BF)
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(g * hacc[i][j][r]), yres,
                                                          off + j * 64, 0, 0);
                  else
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(g * hacc[i][j][r]),
                                                          yres, off + j * 128, 0, 0);
                }
            }
        };
        const bool whole = wcol0 + 64 <= p.N;
        if (p.ybf16) {
          if (whole) rows(std::true_type{}, std::true_type{});
          else rows(std::false_type{}, std::true_type{});
        } else {
          if (whole) rows(std::true_type{}, std::false_type{});
          else rows(std::false_type{}, std::false_type{});
        }
      }
      return;
    }
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto brow = [&](int j) {
    if constexpr (MODE == kGateUpSwiglu) return (j < 2 ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32);
    else return wn * 128 + j * 32;
  };
  // fragment f (0..3 A rows, 4..7 B rows) of K quarter kk
  auto read1 = [&](const u16* sa, const u16* sb, int kk, int f, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
    const int c = kk * 2 + fk;
    if (f < 4)
      af[f] = as_bf16x8(*(const u32x4*)(sa + v3_off(wm * 128 + f * 32 + fr, c)));
    else
      bfr[f - 4] = as_bf16x8(*(const u32x4*)(sb + v3_off(brow(f - 4) + fr, c)));
  };
  // read order A0 B0 B1 B2 B3 A1 A2 A3: MFMAs 0..3 (A0 x B0..B3) need only the
  // first five reads
  constexpr int kRead[8] = {0, 4, 5, 6, 7, 1, 2, 3};
  // MFMA m (0..15) of a quarter: A fragment m/4, B fragment m%4.  Gate/up
  // passes the weight fragment as the MFMA's first operand, so acc holds the
  // transposed 32x32 block: register r of lane (fr, fk) is output column
  // brow(j) + 8*(r/4) + 4*fk + r%4 of tile row wm*128 + i*32 + fr, four
  // consecutive columns of one row per lane and register quad
  auto mfma1 = [&](const bf16x8 (&af)[4], const bf16x8 (&bfr)[4], int m) {
    if constexpr (MODE == kGateUpSwiglu || MODE == kUpRelu)
      acc[m >> 2][m & 3] = mfma32(bfr[m & 3], af[m >> 2], acc[m >> 2][m & 3]);
    else
      acc[m >> 2][m & 3] = mfma32(af[m >> 2], bfr[m & 3], acc[m >> 2][m & 3]);
  };
  bf16x8 fa[4][4], fb[4][4];  // [quarter set][fragment]
  // quarter q: MFMAs on set q; reads for (sa_r, sb_r, kk_r) into set r after
  // its first 8 MFMAs; DMA j0..j0+7 of stage kt_dma (when j0 >= 0) after its
  // even MFMAs
  auto quarter = [&](int q, const u16* sa_r, const u16* sb_r, int kk_r, int r, u16* sa_d,
                     u16* sb_d, int kt_dma, int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      mfma1(fa[q], fb[q], m);
      if (m < 8) read1(sa_r, sb_r, kk_r, kRead[m], fa[r], fb[r]);
      if (j0 >= 0 && (m & 1) == 0) dma(sa_d, sb_d, kt_dma, j0 + (m >> 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto stage = [&](u16* sa, u16* sb, u16* na, u16* nb_, int kt) __attribute__((always_inline)) {
    quarter(0, sa, sb, 2, 2, sa, sb, 0, -1);
    quarter(1, sa, sb, 3, 3, sa, sb, 0, -1);
    wait_vm_lgkm0<0>();  // own reads of this buffer done; stage kt+1 landed
    block_barrier();
    quarter(2, na, nb_, 0, 0, sa, sb, kt + 2, 0);
    quarter(3, na, nb_, 1, 1, sa, sb, kt + 2, 8);
  };
#pragma unroll
  for (int j = 8; j < 16; ++j) dma(sA0, sB0, 0, j);
#pragma unroll
  for (int j = 8; j < 16; ++j) dma(sA1, sB1, 1, j);
#pragma unroll
  for (int j = 0; j < 8; ++j) dma(sA0, sB0, 0, j);
#pragma unroll
  for (int j = 0; j < 8; ++j) dma(sA1, sB1, 1, j);
  // kAtomIn: the tile's kept-cell words and their prefixes ([256 rows][8]
  // each) come in by DMA now, behind the first two stages, so they are in
  // LDS long before the epilogue (entries past the rows or words are masked
  // there); instruction k of wave w fills rows (w*8+k)*8 .. +8
  __shared__ __align__(16) uint32_t s_cells[MODE == kAtomIn ? 4096 : 4];
  if constexpr (MODE == kAtomIn) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int g = wid * 8 + k;
      const int r = g * 8 + (lane >> 3);
      const size_t gi = (size_t)(row0 + min(r, rvalid - 1)) * p.wpr + min(n_tile * 8 + (lane & 7), p.wpr - 1);
      __builtin_amdgcn_global_load_lds(p.bits + gi, (lds_void_t*)(s_cells + g * 64), 4, 0, 0);
      __builtin_amdgcn_global_load_lds(p.bitpre + gi, (lds_void_t*)(s_cells + 2048 + g * 64), 4, 0, 0);
    }
    wait_vm_lgkm0<24>();  // the first stage landed
  } else {
    wait_vm_lgkm0<8>();
  }
  block_barrier();
#pragma unroll
  for (int f = 0; f < 8; ++f) read1(sA0, sB0, 0, f, fa[0], fb[0]);
#pragma unroll
  for (int f = 0; f < 8; ++f) read1(sA0, sB0, 1, f, fa[1], fb[1]);
  for (int kt = 0; kt < nk; kt += 2) {
    stage(sA0, sB0, sA1, sB1, kt);
    stage(sA1, sB1, sA0, sB0, kt + 1);
  }
  wait_vm_lgkm0<0>();

  // kAtomIn: the tile's kept-cell words and their prefixes, [256 rows][8
  // words] each, already in LDS (s_cells, loaded with the first stages); a word
  // past the row's end, or of a row past the tile's rows, is set empty with
  // prefix ksel here; per row the first rank in the tile (rlo)
  // and the tile-local start of its kept cells (rbase, a block scan of the
  // counts); then each word's prefix is turned into the tile-local position of
  // its first kept cell.  Up to kAtomTileCap kept cells of the tile are listed
  // in LDS (fp32 value and row << 8 | column in the tile); a denser tile goes
  // through ukept in global memory instead.
  uint32_t* tbits = s_cells;
  int32_t* tpos = (int32_t*)s_cells + 2048;
  int32_t* rlo = (int32_t*)sB0;
  int32_t* rbase = (int32_t*)sB0 + 256;  // 257 entries
  float* lu = (float*)sA1;
  int32_t* lrc = (int32_t*)sB1;
  bool small_tile = true;
  if constexpr (MODE == kAtomIn) {
    __syncthreads();
    for (int q = tid; q < 2048; q += 256) {
      const int rr = q >> 3, wcol = n_tile * 8 + (q & 7);
      if (!(wcol < p.wpr && rr < rvalid)) {
        tbits[q] = 0u;
        tpos[q] = p.ksel;
      }
    }
    __syncthreads();
    {
      const int r = tid;
      const int lo = r < rvalid ? tpos[r * 8] : 0;
      const int cnt = r < rvalid ? tpos[r * 8 + 7] + __popc(tbits[r * 8 + 7]) - lo : 0;
      int incl = cnt;
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      __shared__ int wtot[4];
      if (lane == 63) wtot[wid] = incl;
      __syncthreads();
      int base = 0;
      for (int w = 0; w < wid; ++w) base += wtot[w];
      rlo[r] = lo;
      rbase[r] = base + incl - cnt;
      if (r == 255) rbase[256] = base + incl;
    }
    __syncthreads();
    small_tile = rbase[256] <= kAtomTileCap;
    if (small_tile) {
      for (int q = tid; q < 2048; q += 256) tpos[q] += rbase[q >> 3] - rlo[q >> 3];
      __syncthreads();
    }
  }

  if constexpr (MODE == kAtomIn) {
    // H = 0 at every cell of the tile (the kept cells are rewritten below, after
    // a barrier); the kept cells' values go to the LDS list (a lane whose cell
    // is not kept writes to its own spare entry, so no branch per cell), or,
    // for a dense tile, to ukept at their rank in the row
    // zeros go through a buffer resource over the tile's rows, so a row past
    // them is dropped by the bounds check; a 32-column group past N (N is a
    // multiple of 32) is skipped by a branch that is uniform over the wave
    const __amdgpu_buffer_rsrc_t hres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.H + (size_t)row0 * p.N), (short)0, rvalid * p.N * 2, 0x00020000);
    const int wcol0 = n_tile * 256 + __builtin_amdgcn_readfirstlane(wn) * 128;
    const uint32_t below = (1u << fr) - 1u;
    const int spare = kAtomTileCap + lane;
    auto cells = [&](auto listed, auto whole) __attribute__((always_inline)) {
      constexpr bool LISTED = decltype(listed)::value;
      constexpr bool WHOLE = decltype(whole)::value;  // all of the wave's 128 columns < N
      // (a row past the tile's rows has empty words: nothing is listed); the
      // next row's words are read one row ahead, before this row's writes
      auto row_of = [&](int t) { return wm * 128 + (t >> 4) * 32 + 8 * ((t & 15) >> 2) + 4 * fk + (t & 3); };
      uint4 wv_n = *(const uint4*)(tbits + row_of(0) * 8 + wn * 4);
      int4 pv_n = *(const int4*)(tpos + row_of(0) * 8 + wn * 4);
#pragma unroll
      for (int t = 0; t < 64; ++t) {
          const int i = t >> 4, r = t & 15;
          const int row = row_of(t);
          const int grow = row0 + row;
          const uint4 wv = wv_n;
          const int4 pv = pv_n;
          if (t + 1 < 64) {
            wv_n = *(const uint4*)(tbits + row_of(t + 1) * 8 + wn * 4);
            pv_n = *(const int4*)(tpos + row_of(t + 1) * 8 + wn * 4);
          }
          const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
          const int ps[4] = {pv.x, pv.y, pv.z, pv.w};
          const int hoff = (row * p.N + n_tile * 256 + wn * 128 + fr) * 2;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (WHOLE || wcol0 + j * 32 < p.N)
              __builtin_amdgcn_raw_buffer_store_b16((u16)0, hres, hoff + j * 64, 0, 0);
            const bool kept = (ws[j] >> fr) & 1u;
            const int pos = ps[j] + __popc(ws[j] & below);
            if constexpr (LISTED) {
              const int at = kept ? pos : spare;
              lu[at] = acc[i][j][r];
              lrc[at] = (row << 8) | (wn * 128 + j * 32 + fr);
            } else if (kept) {  // kept implies row < rvalid
              p.ukept[(size_t)grow * p.ksel + pos] = acc[i][j][r];
            }
          }
        }
    };
    if (small_tile && wcol0 + 128 <= p.N)
      cells(std::true_type{}, std::true_type{});
    else if (small_tile)
      cells(std::true_type{}, std::false_type{});
    else
      cells(std::false_type{}, std::false_type{});
    // the zeros are written before any kept value is (same addresses)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  if constexpr (MODE == kGateUpSwiglu) {
    // the tile's 256 x 128 bf16 outputs are assembled in LDS (rows 0..127 in
    // sA0, 128..255 in sA1; 16-byte chunk c of row r at position c ^ (r & 15)),
    // each lane writing its four consecutive columns as one 8-byte word, and
    // leave in 16-byte stores, 16 lanes per 256-byte row, through a buffer
    // resource that drops rows past the tile's valid ones
    __syncthreads();  // every wave is done with the operand buffers
    auto hq = [&](int row, int chunk) -> u16* {
      return (row < 128 ? sA0 : sA1) + (row & 127) * 128 + ((chunk ^ (row & 15)) << 3);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + fr;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wn * 64 + j * 32 + 8 * q + 4 * fk;
          float h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = silu_f32(acc[i][j][4 * q + e]) * acc[i][j + 2][4 * q + e];
          *(uint2*)(hq(row, col >> 3) + (col & 7)) = make_uint2(pk_bf16(h[0], h[1]), pk_bf16(h[2], h[3]));
        }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t hres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.H + (size_t)row0 * p.N), (short)0, rvalid * p.N * 2, 0x00020000);
    const int c = tid & 15;
    const int col = n_tile * 128 + c * 8;
    u32x4 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = *(const u32x4*)hq(q * 16 + (tid >> 4), c);
    if (col < p.N) {
#pragma unroll
      for (int q = 0; q < 16; ++q)
        __builtin_amdgcn_raw_buffer_store_b128(v[q], hres, ((q * 16 + (tid >> 4)) * p.N + col) * 2, 0, 0);
    }
    return;
  }
  if constexpr (MODE == kDown) {
    // gate-scaled fp32 rows through a buffer resource over the tile's rows of
    // this K slice's output (a row past them is dropped by the bounds check);
    // the row gates come from LDS; in a wave whose 128 columns are not all
    // below N, each lane tests its own column
    __syncthreads();  // every wave is done with the operand buffers
    float* gsc = (float*)sA0;
    gsc[tid] = gpre;
    __syncthreads();
    const int esz = p.ybf16 ? 2 : 4;  // bytes per output element
    const __amdgpu_buffer_rsrc_t yres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)p.Y + ((size_t)ks * p.ystride + (size_t)row0 * p.N) * esz), (short)0,
        rvalid * p.N * esz, 0x00020000);
    const int wcol0 = n_tile * 256 + __builtin_amdgcn_readfirstlane(wn) * 128;
    auto rows = [&](auto whole, auto bf16) __attribute__((always_inline)) {
      constexpr bool WHOLE = decltype(whole)::value;  // all of the wave's 128 columns < N
      constexpr bool BF = decltype(bf16)::value;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
          const float g = gsc[row];
          const int off = (row * p.N + wcol0 + fr) * (BF ? 2 : 4);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (WHOLE || wcol0 + j * 32 + fr < p.N) {
              if constexpr (BF)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(g * acc[i][j][r]), yres,
                                                      off + j * 64, 0, 0);
              else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(g * acc[i][j][r]), yres,
                                                      off + j * 128, 0, 0);
            }
        }
    };
    const bool whole = wcol0 + 128 <= p.N;
    if (p.ybf16) {
      if (whole) rows(std::true_type{}, std::true_type{});
      else rows(std::false_type{}, std::true_type{});
    } else {
      if (whole) rows(std::true_type{}, std::false_type{});
      else rows(std::false_type{}, std::false_type{});
    }
    return;
  }
  if constexpr (MODE == kUpRelu) {
    // as the SwiGLU epilogue (transposed accumulators, four consecutive
    // columns per 8-byte LDS write): the 256 x 256 bf16 tile assembled in LDS
    // (64 rows per 32 KB region; chunk c of row r at position c ^ (r & 31)),
    // then 16-byte buffer stores, 32 lanes per 512-byte row
    __syncthreads();  // every wave is done with the operand buffers
    auto hq = [&](int row, int chunk) -> u16* {
      u16* const reg = row < 128 ? (row < 64 ? sA0 : sA1) : (row < 192 ? sB0 : sB1);
      return reg + (row & 63) * 256 + ((chunk ^ (row & 31)) << 3);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + fr;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wn * 128 + j * 32 + 8 * q + 4 * fk;
          const f32x16& a = acc[i][j];
          *(uint2*)(hq(row, col >> 3) + (col & 7)) =
              make_uint2(pk_bf16(fmaxf(a[4 * q], 0.0f), fmaxf(a[4 * q + 1], 0.0f)),
                         pk_bf16(fmaxf(a[4 * q + 2], 0.0f), fmaxf(a[4 * q + 3], 0.0f)));
        }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t hres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.H + (size_t)row0 * p.N), (short)0, rvalid * p.N * 2, 0x00020000);
    const int c = tid & 31;
    const int col = n_tile * 256 + c * 8;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      u32x4 v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = *(const u32x4*)hq((b * 16 + q) * 8 + (tid >> 5), c);
      if (col < p.N) {
#pragma unroll
        for (int q = 0; q < 16; ++q)
          __builtin_amdgcn_raw_buffer_store_b128(v[q], hres,
                                                 (((b * 16 + q) * 8 + (tid >> 5)) * p.N + col) * 2, 0, 0);
      }
    }
  }

  if constexpr (MODE == kAtomIn) {
    // the tile's kept cells, spread over the block: list entry e of row r has
    // rank rlo[r] + e - rbase[r] in its row, where its gate (and, for a dense
    // tile, its value and column) sit
    __syncthreads();  // the list (or this block's ukept stores) is complete
    const int total = rbase[256];
    if (small_tile) {
      for (int e0 = tid; e0 < total; e0 += 1024) {
        float u[4], g[4];
        int rc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = min(e0 + 256 * q, total - 1);
          rc[q] = lrc[e];
          u[q] = lu[e];
          const int r = rc[q] >> 8;
          g[q] = p.gate[(size_t)(row0 + r) * p.ksel + rlo[r] + e - rbase[r]];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (e0 + 256 * q < total)
            p.H[(size_t)(row0 + (rc[q] >> 8)) * p.N + n_tile * 256 + (rc[q] & 255)] =
                f32_to_bf16(g[q] * silu_f32(u[q]));
      }
    } else {
      for (int e = tid; e < total; e += 256) {
        int lo = 0, hi = 255;  // the last row whose list starts at or before e
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (rbase[mid] <= e)
            lo = mid;
          else
            hi = mid - 1;
        }
        const size_t a = (size_t)(row0 + lo) * p.ksel + rlo[lo] + (e - rbase[lo]);
        p.H[(size_t)(row0 + lo) * p.N + p.kidx[a]] =
            f32_to_bf16(p.gate[a] * silu_f32(p.ukept[a]));
      }
    }
  }
}

template <int MODE>
hipError_t run_tiles_v2(TileArgs a, hipStream_t s) {
  // bound on the real row tiles: sum over experts of ceil(rows_e / 256)
  const int m_tiles_max =
      (a.rows + kV2BM - 1) / kV2BM + (a.E > 1 ? min(a.E, a.rows) : 0);
  a.m_tiles_max = m_tiles_max;
  const int ncols = (MODE == kGateUpSwiglu) ? 128 : 256;
  a.n_tiles = (a.N + ncols - 1) / ncols;
  if (a.ksplit < 1) a.ksplit = 1;
  // each K slice needs an even number of 64-wide stages (callers check K % 128)
  if ((a.K / a.ksplit) % 128 != 0) return hipErrorInvalidValue;
  long long nblk = (long long)m_tiles_max * a.n_tiles * a.ksplit;
  nblk = (nblk + 7) / 8 * 8;
  hipLaunchKernelGGL(grouped_gemm_tile_kernel<MODE>, dim3((unsigned)nblk), dim3(256), 0, s, a);
  return hipGetLastError();
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
  const float u = dot_f32(xr, wur, d);
  float h;
  if (relu) {
    h = fmaxf(u, 0.0f);
  } else {
    const float g = dot_f32(xr, wg + ((size_t)e * F + f) * d, d);
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
  const float s = dot_f32(hr, wr, F);
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
  // the dynamic-LDS limit is raised once per device for this instantiation,
  // under a lock, so concurrent first calls from several threads are safe
  static std::mutex attr_mu;
  static bool attr_set[kAttrDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lk(attr_mu);
    const bool cached = dev >= 0 && dev < kAttrDevices;
    if (!cached || !attr_set[dev]) {
      e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
      if (e != hipSuccess) return e;
      if (cached) attr_set[dev] = true;
    }
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

bool ffn_rows_bf16_applies(const FfnProblem& p) {
  // the 256x256 down path of the tiled launch with dense bf16 experts
  return p.dt == MOE_DT_BF16 && p.w && !p.w->q_up && !stream_ffn_applies(p) && p.F % 128 == 0;
}

bool ffn_direct_applies(const FfnProblem& p) {
  if (p.offsets && !p.row_assign) return false;
  return stream_ffn_applies(p) && p.k <= 2 && p.down_splits <= 1;
}

size_t ffn_ws_bytes(int rows, int F, moe_dtype dt) {
  return (size_t)rows * F * (dt == MOE_DT_F32 ? 4 : 2);
}

int ffn_down_splits(int T, int d, int F, int E, int k, moe_dtype dt, const moe_experts* w) {
  const bool int4 = w && w->q_up;
  if (dt != MOE_DT_BF16 || T <= 0) return 1;
  FfnProblem q{};
  q.T = T; q.d = d; q.F = F; q.dt = dt; q.rows = T * k; q.w = w;
  if (int4) {
    // weight streaming: K parts of the row-split down kernel
    if (!stream_ffn_applies(q) || !w->q_down) return 1;
    const int P = stream_down_parts(d, F, E);
    return (P > 1 && stream_rows_applies(F, P, w->q_down, w->q_down)) ? P : 1;
  }
  if (stream_ffn_applies(q)) return 1;
  // tiles of one slice (upper bound, as the launcher sizes the grid), in rounds
  // of one tile per CU (256 CUs); a slice costs 1/S of a full-K tile, and each
  // extra slice adds a partial-row write and read (charged as 0.1 round)
  constexpr int kCUs = 256;
  const int rows = T * k;
  const long long tiles = (long long)((rows + kV2BM - 1) / kV2BM + min(E, rows)) * ((d + 255) / 256);
  int best = 1;
  double best_cost = 1e30;
  for (int S = 1; S <= 4; S *= 2) {
    if (F % (128 * S) != 0) break;
    const double cost = (double)((tiles * S + kCUs - 1) / kCUs) / S + 0.1 * (S - 1);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

hipError_t launch_grouped_ffn(const FfnProblem& p, hipStream_t s, hipEvent_t mid) {
  if (p.rows == 0) return hipSuccess;
  if (p.y_direct && !ffn_direct_applies(p)) return hipErrorInvalidValue;
  if (p.xw && stream_ffn_applies(p)) return hipErrorInvalidValue;  // tiled path only
  if (stream_ffn_applies(p)) return launch_stream_ffn(p, s, mid);
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
  const bool v2_gu = !int4 && (p.d % 128 == 0);
  if (p.xw) {
    // the extra slot runs only on the 256x256 path
    if (int4 || !v2_gu || p.F % 128 != 0 || p.xw->q_up) return hipErrorInvalidValue;
    a.xB0 = (const u16*)(relu ? p.xw->w_up : p.xw->w_gate);
    a.xB1 = (const u16*)p.xw->w_up;
    a.xslot = p.xslot;
  }
  if (relu)
    e = int4 ? run_tiles<128, 128, kUpRelu, true>(a, s)
             : (v2_gu ? run_tiles_v2<kUpRelu>(a, s) : run_tiles<128, 128, kUpRelu, false>(a, s));
  else
    e = int4 ? run_tiles<128, 128, kGateUpSwiglu, true>(a, s)
             : (v2_gu ? run_tiles_v2<kGateUpSwiglu>(a, s)
                      : run_tiles<128, 128, kGateUpSwiglu, false>(a, s));
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
  b.ksplit = p.down_splits > 1 ? p.down_splits : 1;
  b.ystride = (size_t)p.rows * p.d;
  if (int4) {
    b.q0 = p.w->q_down->q; b.s0 = p.w->q_down->scale; b.z0 = p.w->q_down->zero;
    return run_tiles<128, 128, kDown, true>(b, s);
  }
  b.B0 = (const u16*)p.w->w_down;
  if (p.rows_bf16) {
    if (!ffn_rows_bf16_applies(p)) return hipErrorInvalidValue;
    b.ybf16 = 1;
  }
  if (p.xw) {
    b.xB0 = (const u16*)p.xw->w_down;
    b.xslot = p.xslot;
  }
  if (p.F % 128 == 0) return run_tiles_v2<kDown>(b, s);
  if (b.ksplit > 1) return hipErrorInvalidValue;  // slices exist only on the 256x256 path
  return run_tiles<128, 128, kDown, false>(b, s);
}

hipError_t launch_gemm_bt(const u16* A, int lda, int M, const u16* B, int N, int K, float* Y,
                          int ksplit, size_t ystride, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (K % (128 * (ksplit < 1 ? 1 : ksplit)) != 0) return hipErrorInvalidValue;
  TileArgs a = {};
  a.A = A;
  a.lda = lda;
  a.B0 = B;
  a.N = N;
  a.K = K;
  a.E = 1;
  a.rows = M;
  a.Y = Y;
  a.ksplit = ksplit < 1 ? 1 : ksplit;
  a.ystride = ystride;
  return run_tiles_v2<kDown>(a, s);
}

hipError_t launch_atomic_in(const u16* A, int M, const u16* B, int N, int K, const uint32_t* bits,
                            const int32_t* bitpre, const int32_t* kidx, const float* gates,
                            int ksel, float* ukept, u16* H, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (K % 128 != 0 || N % 32 != 0) return hipErrorInvalidValue;
  TileArgs a = {};
  a.A = A;
  a.lda = K;
  a.B0 = B;
  a.N = N;
  a.K = K;
  a.E = 1;
  a.rows = M;
  a.H = H;
  a.ukept = ukept;
  a.kidx = kidx;
  a.gate = gates;
  a.bits = bits;
  a.bitpre = bitpre;
  a.wpr = N / 32;
  a.ksel = ksel;
  a.ksplit = 1;
  return run_tiles_v2<kAtomIn>(a, s);
}

}  // namespace moe
