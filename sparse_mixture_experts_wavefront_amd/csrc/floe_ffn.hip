// floe_ffn.hip -- contextual sparse down-projection for decode.
//
// "FloE: On-the-Fly MoE Inference on Memory-constrained GPU" -- Core claim and
// What carries the argument: in an expert's hidden layer, channels whose
// up-projection output is small in magnitude are pruned per token; a pruned
// channel needs neither its gate row nor its down-projection column, and the up
// projection that decides it is stored in INT2.  One threshold per expert.
//
// Per layer call (rows grouped by expert):
//   1. INT2 up projection of every row (the nested-weight kernel in its up mode,
//      mwq_ffn.hip): U [rows][F] fp32 and, per expert and channel, whether some
//      row of the expert has |U| > threshold.
//   2. floe_compact_kernel: per expert, the list of those channels, ascending.
//   3. floe_gate_kernel: gate rows of the listed channels only (a gather of
//      whole contiguous rows), 16x16x32 MFMA against the expert's token rows;
//      h = bf16(silu(g) * u) where the row's own |u| passes, else 0, stored in
//      list order (Hc).
//   4. floe_down_kernel: the down projection over the listed channels only,
//      W_down stored transposed so a channel is one contiguous row of d_model
//      values.  With a few token rows per expert this is a sparse GEMV: each
//      lane owns four output columns and runs fp32 FMAs over the channels, the
//      hidden values broadcast from LDS; the channel list is split into slices
//      whose partial sums the combine adds in a fixed order.
// A row keeps exactly its own channels: a channel that only another row of the
// same expert keeps has h = 0 for this row, so the union only sets what is read.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGateChMax = 32;  // listed channels per gate block (16 or 32)
constexpr int kDownCols = 1024; // output columns per down block (4 per lane)
constexpr int kDownJc = 64;     // channels staged in LDS per down step
constexpr int kCompactSeg = 128;  // flags per thread of the list kernel (d_ff <= 32768)

// ---- 2. per-expert list of kept channels ------------------------------------
// Thread tid owns a segment of seg flags (a multiple of 8, read as 8-byte words;
// flags are 0 or 1 bytes, so a word's popcount is its number of kept channels);
// a wave-level and then a block-level exclusive scan of the segment counts
// gives each thread its output position.
__global__ __launch_bounds__(256) void floe_compact_kernel(const int32_t* __restrict__ offsets,
                                                           const uint8_t* __restrict__ flags,
                                                           int F, int32_t* __restrict__ list,
                                                           int32_t* __restrict__ nnz) {
  __shared__ int wsum[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (offsets[e + 1] - offsets[e] <= 0) {  // no rows: the up pass left no flags
    if (tid == 0) nnz[e] = 0;
    return;
  }
  const int seg = (((F + 255) / 256) + 7) & ~7;  // <= kCompactSeg (F <= 32768)
  const int f0 = min(tid * seg, F), f1 = min(f0 + seg, F);
  const uint8_t* fl = flags + (size_t)e * F;
  // the segment's flag words, all loads issued before the first use
  uint2 v[kCompactSeg / 8];
#pragma unroll
  for (int i = 0; i < kCompactSeg / 8; ++i)
    v[i] = f0 + 8 * i < f1 ? *(const uint2*)(fl + f0 + 8 * i) : make_uint2(0u, 0u);
  int c = 0;
#pragma unroll
  for (int i = 0; i < kCompactSeg / 8; ++i) c += __popc(v[i].x) + __popc(v[i].y);
  // inclusive scan inside the wave, then across the 4 waves
  int incl = c;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wv; ++w) base += wsum[w];
  int pos = base + incl - c;
  int32_t* out = list + (size_t)e * F;
#pragma unroll
  for (int i = 0; i < kCompactSeg / 8; ++i)
#pragma unroll
    for (int b = 0; b < 8; ++b)
      if (((b < 4 ? v[i].x : v[i].y) >> (8 * (b & 3))) & 1u) out[pos++] = f0 + 8 * i + b;
  if (tid == 255) nnz[e] = base + incl;
}

// ---- 3. gate rows of the listed channels -----------------------------------
struct GateArgs {
  const u16* X;            // x [T][K]
  const int32_t* gather;   // row -> flat assignment (token = a / k)
  int k;
  const u16* Wg;           // [E][F][K]
  int F, K;
  const int32_t* offsets;  // [E+1]
  const int32_t* list;     // [E][F]
  const int32_t* nnz;      // [E]
  const float* U;          // [rows][F]
  const float* thr;        // [E]
  u16* Hc;                 // [rows][F], column j = j-th listed channel
  int E;                   // experts (E <= 64)
};

// Work items are chunks of CH consecutive listed channels, numbered over the
// experts in id order (an expert without rows has none); blocks take chunks
// blockIdx.x, + gridDim.x, ... so the grid is sized to the chip, not to the
// largest possible list.  Each wave owns a quarter of K; lane (r, g) feeds MFMA
// step s with K values [s*32 + g*8, +8) of an iteration of 128 (channel row r
// of its 16-row block, token row r of the B operand), loads D iterations ahead.
template <int CH, int D>
__global__ __launch_bounds__(256) void floe_gate_kernel(GateArgs p) {
  constexpr int RB = CH / 16, NS = 4;
  __shared__ f32x4 red[4][RB][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // chunk counts per expert (lane = expert), inclusive scan over the wave
  int nch = 0;
  if (lane < p.E && p.offsets[lane + 1] > p.offsets[lane]) nch = (p.nnz[lane] + CH - 1) / CH;
  int incl = nch;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const int total = __shfl(incl, 63, 64);
  const int r16 = lane & 15, g = lane >> 4;
  const int Kq = p.K >> 2, kw0 = w * Kq, iters = Kq / 128;
  for (int ci = blockIdx.x; ci < total; ci += gridDim.x) {
    const int e = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(incl > ci)));
    const int j0 = __builtin_amdgcn_readfirstlane((ci - __shfl(incl - nch, e, 64)) * CH);
    const int nz = __builtin_amdgcn_readfirstlane(p.nnz[e]);
    const int row0 = __builtin_amdgcn_readfirstlane(p.offsets[e]);
    const int cnt = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]) - row0;
    const int32_t* lst = p.list + (size_t)e * p.F;
    const u16* wrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int j = min(j0 + rb * 16 + r16, nz - 1);  // past the list: a listed row, unused
      wrow[rb] = p.Wg + ((size_t)e * p.F + lst[j]) * p.K + kw0 + g * 8;
    }
    for (int mbase = 0; mbase < cnt; mbase += 16) {
      const int mrows = min(16, cnt - mbase);
      const int tr = row0 + mbase + min(r16, mrows - 1);
      const u16* xr = p.X + (size_t)(p.gather[tr] / p.k) * p.K + kw0 + g * 8;
      struct Set {
        u32x4 w[RB][NS];
        u32x4 x[NS];
      };
      auto load = [&](Set& S, int it) __attribute__((always_inline)) {
        it = min(it, iters - 1);  // past the end: reload the last iteration (unused)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int s = 0; s < NS; ++s) S.w[rb][s] = *(const u32x4*)(wrow[rb] + it * 128 + s * 32);
        // token lanes past the pass's rows take zeros and fetch nothing
        if (r16 < mrows) {
#pragma unroll
          for (int s = 0; s < NS; ++s) S.x[s] = *(const u32x4*)(xr + it * 128 + s * 32);
        } else {
#pragma unroll
          for (int s = 0; s < NS; ++s) S.x[s] = u32x4{0u, 0u, 0u, 0u};
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      f32x4 acc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      Set st[D];
#pragma unroll
      for (int u = 0; u < D; ++u) load(st[u], u);
      for (int it0 = 0; it0 < iters; it0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
          if (it0 + u < iters) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int rb = 0; rb < RB; ++rb)
                acc[rb] = mfma16(as_bf16x8(st[u].w[rb][s]), as_bf16x8(st[u].x[s]), acc[rb]);
          }
          load(st[u], it0 + u + D);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) red[w][rb][lane] = acc[rb];
      __syncthreads();
      for (int o = tid; o < 16 * CH; o += 256) {
        const int m = o / CH, col = o % CH;
        const int j = j0 + col;
        if (mbase + m >= cnt || j >= nz) continue;
        // C layout of the 16x16 MFMA: channel row 4*(lane/16)+i, token column lane%16
        const int rb = col >> 4, rr = col & 15;
        const int ln = (rr >> 2) * 16 + m, i = rr & 3;
        float gv = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) gv += red[ww][rb][ln][i];
        const size_t orow = (size_t)(row0 + mbase + m);
        const float u = p.U[orow * p.F + lst[j]];
        p.Hc[orow * p.F + j] = fabsf(u) > p.thr[e] ? f32_to_bf16(silu_f32(gv) * u) : (u16)0;
      }
    }
  }
}

// ---- 4. down projection over the listed channels ----------------------------
struct DownArgs {
  const u16* Hc;           // [rows][F]
  const u16* WdT;          // [E][F][d]
  int F, d;
  const int32_t* offsets;  // [E+1]
  const int32_t* list;     // [E][F]
  const int32_t* nnz;      // [E]
  const int32_t* gate_map; // row -> flat assignment
  const float* gate;
  float* Y;                // [S][rows][d]
  int S, ncc, rows;
  int E;                   // experts (E <= 64)
};

// Block (expert with rows, 1024-column chunk, channel slice), experts with rows
// numbered in id order so the grid covers only as many as the call can have;
// lane owns 4 consecutive
// output columns (one 8-byte load per channel) and runs fp32 FMAs over the
// slice's channels, 8 at a time, the hidden values of up to MR token rows
// broadcast from LDS.
__global__ __launch_bounds__(256) void floe_down_kernel(DownArgs p) {
  constexpr int U = 8;
  __shared__ __align__(16) float hs[16][kDownJc];
  __shared__ int chs[kDownJc];
  const int tid = threadIdx.x;
  const int s = blockIdx.x % p.S;
  const int cc = (blockIdx.x / p.S) % p.ncc;
  const int e = __builtin_amdgcn_readfirstlane(
      active_expert(p.offsets, 1, p.E, blockIdx.x / (p.S * p.ncc)));
  if (e < 0) return;
  const int row0 = __builtin_amdgcn_readfirstlane(p.offsets[e]);
  const int cnt = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]) - row0;
  if (cnt <= 0) return;
  const int nz = __builtin_amdgcn_readfirstlane(p.nnz[e]);
  const int L = (nz + p.S - 1) / p.S;
  const int jb = min(s * L, nz), je = min(jb + L, nz);
  // d is a multiple of 512, so the last chunk may be half used: lanes past d
  // load the chunk's last 4 columns again and store nothing
  const int col = cc * kDownCols + 4 * tid;
  const int lcol = min(col, p.d - 4);
  const int32_t* lst = p.list + (size_t)e * p.F;
  const u16* wbase = p.WdT + (size_t)e * p.F * p.d + lcol;

  auto body = [&](auto mrc, int mbase) __attribute__((always_inline)) {
    constexpr int MR = decltype(mrc)::value;  // rows per pass held in registers
    const int mrows = min(MR, cnt - mbase);
    float a[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) a[m][c] = 0.0f;
    for (int jc = jb; jc < je; jc += kDownJc) {
      const int n = min(kDownJc, je - jc);
      __syncthreads();
      for (int i = tid; i < MR * kDownJc; i += 256) {
        const int m = i / kDownJc, jj = i - m * kDownJc;
        float hv = 0.0f;
        if (jj < n && m < mrows) hv = bf16_to_f32(p.Hc[(size_t)(row0 + mbase + m) * p.F + jc + jj]);
        hs[m][jj] = hv;
        if (m == 0) chs[jj] = lst[jc + min(jj, n - 1)];
      }
      __syncthreads();
      // U channels per step (a partial last step reads listed rows with h = 0)
      for (int jj = 0; jj < n; jj += U) {
        uint2 wv[U];
#pragma unroll
        for (int q = 0; q < U; ++q) wv[q] = *(const uint2*)(wbase + (size_t)chs[jj + q] * p.d);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const f32x4 h0 = *(const f32x4*)&hs[m][jj];
          const f32x4 h1 = *(const f32x4*)&hs[m][jj + 4];  // jj + 8 <= kDownJc
#pragma unroll
          for (int q = 0; q < U; ++q) {
            const float h = q < 4 ? h0[q] : h1[q - 4];
            a[m][0] = fmaf(h, __uint_as_float(wv[q].x << 16), a[m][0]);
            a[m][1] = fmaf(h, __uint_as_float(wv[q].x & 0xffff0000u), a[m][1]);
            a[m][2] = fmaf(h, __uint_as_float(wv[q].y << 16), a[m][2]);
            a[m][3] = fmaf(h, __uint_as_float(wv[q].y & 0xffff0000u), a[m][3]);
          }
        }
      }
    }
    if (col < p.d) {
      for (int m = 0; m < mrows; ++m) {
        const size_t orow = (size_t)(row0 + mbase + m);
        const float gs = p.gate ? p.gate[p.gate_map[orow]] : 1.0f;
        float* yo = p.Y + ((size_t)s * p.rows + orow) * p.d + col;
        *(float4*)yo = make_float4(gs * a[m][0], gs * a[m][1], gs * a[m][2], gs * a[m][3]);
      }
    }
  };
  // registers for exactly as many rows as the pass has (up to 16): every FMA
  // beyond them would be wasted work
  for (int mbase = 0; mbase < cnt; mbase += 16) {
    const int r = cnt - mbase;
    if (r <= 1)
      body(std::integral_constant<int, 1>{}, mbase);
    else if (r <= 2)
      body(std::integral_constant<int, 2>{}, mbase);
    else if (r <= 4)
      body(std::integral_constant<int, 4>{}, mbase);
    else if (r <= 8)
      body(std::integral_constant<int, 8>{}, mbase);
    else
      body(std::integral_constant<int, 16>{}, mbase);
  }
}

}  // namespace

int floe_down_splits(int d, int E) {
  // about 2048 blocks over the experts and 1024-column chunks, at most 32 slices
  const int base = E * ((d + kDownCols - 1) / kDownCols);
  int S = base > 0 ? 2048 / base : 1;
  return S < 1 ? 1 : (S > 32 ? 32 : S);
}

const char* floe_unsupported(int T, int d, int F, int k) {
  if (const char* why = mwq_ffn_unsupported(T, d, F, k)) return why;
  if (F % kGateChMax != 0) return "sparse down-projection needs d_ff a multiple of 32";
  if (F > 256 * kCompactSeg) return "sparse down-projection needs d_ff <= 32768";
  return nullptr;
}

hipError_t launch_floe_ffn(const FloeProblem& p, hipStream_t s, hipEvent_t mid) {
  if (floe_unsupported(p.T, p.d, p.F, p.k)) return hipErrorInvalidValue;
  hipError_t e = launch_int2_up(p.x, p.T, p.d, p.F, p.E, p.k, p.w->up, p.offsets, p.row_assign,
                                p.w->threshold, p.U, p.flags, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(floe_compact_kernel, dim3(p.E), dim3(256), 0, s, p.offsets, p.flags, p.F,
                     p.list, p.nnz);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  GateArgs g{};
  g.X = (const u16*)p.x;
  g.gather = p.row_assign;
  g.k = p.k;
  g.Wg = (const u16*)p.w->w_gate;
  g.F = p.F;
  g.K = p.d;
  g.offsets = p.offsets;
  g.list = p.list;
  g.nnz = p.nnz;
  g.U = p.U;
  g.thr = p.w->threshold;
  g.Hc = p.Hc;
  // few rows (a one- or two-token step): few experts are active, so narrower
  // blocks, each with more loads in flight, give the gather more of them
  g.E = p.E;
  const int eact = p.rows < p.E ? p.rows : p.E;  // experts that can have rows
  if (p.rows <= 4) {
    const int grid = std::min(eact * (p.F / 16), 512);
    hipLaunchKernelGGL((floe_gate_kernel<16, 4>), dim3(grid), dim3(256), 0, s, g);
  } else {
    const int grid = std::min(eact * (p.F / 32), 2048);
    hipLaunchKernelGGL((floe_gate_kernel<32, 2>), dim3(grid), dim3(256), 0, s, g);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (mid) {
    e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
  }
  DownArgs dn{};
  dn.Hc = p.Hc;
  dn.WdT = (const u16*)p.w->w_down_t;
  dn.F = p.F;
  dn.d = p.d;
  dn.offsets = p.offsets;
  dn.list = p.list;
  dn.nnz = p.nnz;
  dn.gate_map = p.row_assign;
  dn.gate = p.gate;
  dn.Y = p.y_rows;
  dn.S = p.splits;
  dn.ncc = (p.d + kDownCols - 1) / kDownCols;
  dn.rows = p.rows;
  dn.E = p.E;
  hipLaunchKernelGGL(floe_down_kernel, dim3(eact * dn.ncc * dn.S), dim3(256), 0, s, dn);
  return hipGetLastError();
}

}  // namespace moe
