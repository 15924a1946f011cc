// mwq_ffn.hip -- grouped expert FFN on nested (matryoshka) 2/3/4-bit weights.
//
// "D^2MoE: Dual Routing and Dynamic Scheduling for Efficient On-Device
// MoE-based LLM Serving" -- What carries the argument (the 2-bit weights nest in
// the 3-bit ones and those in the 4-bit ones; each (token, expert) pair runs at
// its own width) and Figure 8 (the low-bit weights are decoded inside the GEMM
// kernel).  A weight at width b decodes as (the format of include/moe.h):
//   w = fp32(fp32(q) - z2) * s2;  b >= 3: w = w + (r3 ? a3 : -a3);
//   b == 4: w = w + (r4 ? a4 : -a4);  W = bf16_RNE(w)
// Inside one group of 128 weights of one row, W is a function of the code
// (q, r3, r4) alone: 4 values at width 2, 8 at width 3, 16 at width 4.  So the
// kernel decodes by table.  Per row and group, a lane computes the tables with
// the fp32 steps above (at most 28 values), rounds them to bf16 and splits each
// table into a low-byte and a high-byte part; four weights are then looked up
// per v_perm_b32 with byte-sized codes as selectors.  The byte-transposed
// storage order gives those codes with one shift and one mask per four
// consecutive weights (a residual bit adds one shift and one and-or), and two
// more byte permutes interleave the low and high bytes into two packed bf16
// pairs in K order, ready for the MFMA.  Width 4 has 16 entries, more than one
// v_perm_b32 reaches: two lookups (r4 = 0 and r4 = 1 halves) and a byte select.
//
// One block = one expert x a strip of 32 output columns (64 weight rows for
// gate/up: 32 gate + 32 up, the same columns), all of the expert's rows and
// all widths: codes and residual bits are read once, each width present among
// the rows of a pass gets its own lookups and MFMAs into its own accumulator,
// and the epilogue takes, per token row, the accumulator of that row's width.
// The 4 waves split K in 512-wide iterations; inside one, lane (r, g) owns
// weight row r of its 16-row block and group g (128 weights), so it builds
// tables once per iteration.  Sub-step u covers K [u*32, +32) of that group in
// 4 MFMA steps (16x16x32, fp32 accumulate); its codes, residual bits and token
// operands are loaded two sub-steps ahead through buffer resources, and a
// sub-step past the wave's K range reads past the resource, which returns zeros
// without touching memory.  Token rows run in passes of 16 (a decode step
// gives each expert a few rows); each pass re-reads the strip.  The 4 waves'
// partial sums meet in LDS, where the epilogue applies SiLU(gate) * up (to bf16
// H) or the gate scale (fp32 rows), as in the bf16 and INT4 kernels.
#include <type_traits>

#include "moe_internal.h"

#ifndef MWQ_WAVES
#define MWQ_WAVES 3
#endif
#ifndef MWQ_RM_GU
#define MWQ_RM_GU 16
#endif
#ifndef MWQ_RM_DN
#define MWQ_RM_DN 32
#endif

namespace moe {
namespace {

// kMModeUp: one INT2 matrix (the width-2 base alone), fp32 outputs U and, per
// output column, whether any row of the expert exceeds the expert's threshold in
// magnitude (the channel flags of the contextual sparse down-projection)
constexpr int kMModeGateUp = 0, kMModeRelu = 1, kMModeDown = 2, kMModeUp = 3;

struct MwqArgs {
  const u16* X;            // gate/up: x [T][ldx]; down: H [rows][ldx]
  int ldx;
  const int32_t* gather;   // gate/up: row -> flat assignment (token = a / k); down: NULL
  int k;
  moe_wmwq W0, W1;         // gate/up: gate, up (ReLU: W_in in W0); down: W_down in W0
  int N, K;
  const int32_t* offsets;  // [gpe*E+1], group gpe*e + j = expert e at width 2 + j
  int gpe;                 // groups per expert: 3 (nested widths) or 1 (INT2 only)
  float* U;                // up mode: output [rows][N] fp32
  const float* thr;        // up mode: [E] magnitude thresholds
  uint8_t* flags;          // up mode: [E][N] 1 where a row of the expert keeps the channel
  u16* H;                  // gate/up output [rows][N]
  float* Y;                // down output [rows][N]
  const int32_t* gate_map; // down: row -> flat assignment (gate index)
  const float* gate;
  int nblk_per_expert;
  int E;                   // experts (E <= 64)
  uint32_t xbytes;         // bytes of X (buffer resource size)
};

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  // byte j of the result = byte sel.j of the 8-byte value hi:lo (0..3 from lo)
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// low / high bytes of the four bf16 values in the packed pairs (e0,e1), (e2,e3)
__device__ __forceinline__ uint32_t lo_bytes(uint32_t p01, uint32_t p23) {
  return perm(p23, p01, 0x06040200u);
}
__device__ __forceinline__ uint32_t hi_bytes(uint32_t p01, uint32_t p23) {
  return perm(p23, p01, 0x07050301u);
}

// Decode tables of one row and group, bf16 split into low and high bytes;
// byte c of a table part holds entry c (of the part's four).
struct Tab {
  uint32_t l2, h2;          // width 2: entry q
  uint32_t l3[2], h3[2];    // width 3: entry q + 4*r3
  uint32_t l4[4], h4[4];    // width 4: entry q + 4*r3 + 8*r4
};

// md.x = s2 | z2 << 16, md.y = a3 | a4 << 16 (fp16 bits); WM: widths needed
// (bit 0: 2, bit 1: 3, bit 2: 4)
template <int WM>
__device__ __forceinline__ void build_tab(Tab& t, uint2 md) {
  const float s = h2f((u16)(md.x & 0xffffu)), z = h2f((u16)(md.x >> 16));
  const float a3 = h2f((u16)(md.y & 0xffffu)), a4 = h2f((u16)(md.y >> 16));
  float w2[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) w2[q] = __fmul_rn(__fsub_rn((float)q, z), s);
  if constexpr ((WM & 1) != 0) {
    const uint32_t p01 = pk_bf16(w2[0], w2[1]), p23 = pk_bf16(w2[2], w2[3]);
    t.l2 = lo_bytes(p01, p23);
    t.h2 = hi_bytes(p01, p23);
  }
  if constexpr ((WM & 6) != 0) {
    float w3[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) w3[c] = __fadd_rn(w2[c & 3], (c & 4) ? a3 : -a3);
    if constexpr ((WM & 2) != 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t p01 = pk_bf16(w3[4 * h], w3[4 * h + 1]);
        const uint32_t p23 = pk_bf16(w3[4 * h + 2], w3[4 * h + 3]);
        t.l3[h] = lo_bytes(p01, p23);
        t.h3[h] = hi_bytes(p01, p23);
      }
    }
    if constexpr ((WM & 4) != 0) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float w4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 4 * h + j;
          w4[j] = __fadd_rn(w3[c & 7], (c & 8) ? a4 : -a4);
        }
        const uint32_t p01 = pk_bf16(w4[0], w4[1]), p23 = pk_bf16(w4[2], w4[3]);
        t.l4[h] = lo_bytes(p01, p23);
        t.h4[h] = hi_bytes(p01, p23);
      }
    }
  }
}

// packed bf16 pairs (weights 0,1) and (2,3) from the low and high bytes
__device__ __forceinline__ uint32_t pair01(uint32_t L, uint32_t H) { return perm(H, L, 0x05010400u); }
__device__ __forceinline__ uint32_t pair23(uint32_t L, uint32_t H) { return perm(H, L, 0x07030602u); }

// RM: output columns per block (weight rows per matrix in a block)
template <int MODE, int RM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MWQ_WAVES, 8)))
void mwq_stream_kernel(MwqArgs p) {
  constexpr int R = (MODE == kMModeGateUp) ? 2 * RM : RM;  // weight rows per block
  constexpr int RB = R / 16;
  constexpr int NOUT = RM;

  extern __shared__ __align__(16) unsigned char smem[];
  float* red = (float*)smem;                           // [4][RB][64][4]
  uint2* md = (uint2*)(smem + 4 * RB * 64 * 16);       // [R][G+1]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ai = blockIdx.x / p.nblk_per_expert;
  const int nb = blockIdx.x - ai * p.nblk_per_expert;
  const int e = __builtin_amdgcn_readfirstlane(active_expert(p.offsets, p.gpe, p.E, ai));
  if (e < 0) return;
  const int* off = p.offsets + p.gpe * e;
  const int row0 = __builtin_amdgcn_readfirstlane(off[0]);
  const int cnt = __builtin_amdgcn_readfirstlane(off[p.gpe]) - row0;
  // first width-3 and width-4 rows (one group per expert: every row at width 2)
  const int b3 = p.gpe == 3 ? __builtin_amdgcn_readfirstlane(off[1]) - row0 : cnt;
  const int b4 = p.gpe == 3 ? __builtin_amdgcn_readfirstlane(off[2]) - row0 : cnt;
  if (cnt <= 0) return;
  __shared__ int uflag[RM];  // up mode: per output column, some row kept it
  if constexpr (MODE == kMModeUp) {
    if (tid < RM) uflag[tid] = 0;
  }
  const int n0 = nb * NOUT;
  const int r16 = lane & 15, g = lane >> 4;
  const int NI = p.K >> 9;              // 512-wide K iterations
  const int ipw = (NI + 3) >> 2;        // iterations per wave
  const int nsub = ipw * 4;             // sub-steps per wave
  const int G = p.K >> 7, GP = G + 1;
  const uint32_t qrow = (uint32_t)p.K / 4, prow = (uint32_t)p.K / 8;  // bytes per row

  // group metadata of the block's rows into LDS, md[r][g] = {s2 | z2 << 16,
  // a3 | a4 << 16}: block row r < RM is row n0 + r of W0, r >= RM (gate/up) row
  // n0 + r - RM of W1.  Four groups per 8-byte load (G is a multiple of 4).
  auto stage_md = [&]() __attribute__((always_inline)) {
    const int G4 = G >> 2;
    for (int i = tid; i < R * G4; i += 256) {
      const int r = i / G4, c = i - r * G4;
      const bool second = (MODE == kMModeGateUp) && r >= RM;
      const size_t o = ((size_t)e * p.N + n0 + (r % RM)) * G + 4 * c;
      const uint2 vs = *(const uint2*)((second ? p.W1.s2 : p.W0.s2) + o);
      const uint2 vz = *(const uint2*)((second ? p.W1.z2 : p.W0.z2) + o);
      // INT2-only weights have no residual magnitudes
      const u16* a3 = second ? p.W1.a3 : p.W0.a3;
      const u16* a4 = second ? p.W1.a4 : p.W0.a4;
      const uint2 v3 = a3 ? *(const uint2*)(a3 + o) : make_uint2(0u, 0u);
      const uint2 v4 = a4 ? *(const uint2*)(a4 + o) : make_uint2(0u, 0u);
      uint2* dst = md + r * GP + 4 * c;
      // entry j: the low (j even) or high (j odd) halves of word j / 2
      dst[0] = make_uint2(perm(vz.x, vs.x, 0x05040100u), perm(v4.x, v3.x, 0x05040100u));
      dst[1] = make_uint2(perm(vz.x, vs.x, 0x07060302u), perm(v4.x, v3.x, 0x07060302u));
      dst[2] = make_uint2(perm(vz.y, vs.y, 0x05040100u), perm(v4.y, v3.y, 0x05040100u));
      dst[3] = make_uint2(perm(vz.y, vs.y, 0x07060302u), perm(v4.y, v3.y, 0x07060302u));
    }
  };

  // buffer resources over the block's RM-row strips (sizes checked on the host
  // to fit 32-bit offsets)
  const size_t rbase = (size_t)e * p.N + n0;
  const uint32_t qstrip = (uint32_t)RM * qrow, pstrip = (uint32_t)RM * prow;
  auto rsrc = [](const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
  };
  const moe_wmwq& M1 = (MODE == kMModeGateUp) ? p.W1 : p.W0;
  const __amdgpu_buffer_rsrc_t rq0 = rsrc((const char*)p.W0.q2 + rbase * qrow, qstrip);
  const __amdgpu_buffer_rsrc_t rq1 = rsrc((const char*)M1.q2 + rbase * qrow, qstrip);
  const __amdgpu_buffer_rsrc_t r30 = rsrc((const char*)p.W0.p3 + rbase * prow, pstrip);
  const __amdgpu_buffer_rsrc_t r31 = rsrc((const char*)M1.p3 + rbase * prow, pstrip);
  const __amdgpu_buffer_rsrc_t r40 = rsrc((const char*)p.W0.p4 + rbase * prow, pstrip);
  const __amdgpu_buffer_rsrc_t r41 = rsrc((const char*)M1.p4 + rbase * prow, pstrip);
  const __amdgpu_buffer_rsrc_t xres = rsrc(p.X, p.xbytes);
  // lane offsets inside the strips: row (rb*16 + r16) % RM, group g of the iteration
  uint32_t qoff[RB], poff[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint32_t rr = (uint32_t)((rb * 16 + r16) % RM);
    qoff[rb] = rr * qrow + (uint32_t)g * 32u;
    poff[rb] = rr * prow + (uint32_t)g * 16u;
  }

  auto pass = [&](auto wmc, int mbase) __attribute__((always_inline)) {
    constexpr int WM = decltype(wmc)::value;
    const int mrows = min(16, cnt - mbase);
    const int tr = row0 + mbase + min(r16, mrows - 1);  // rows past the count: clamped (no load)
    const int src = p.gather ? p.gather[tr] / p.k : tr;
    const uint32_t xoff = ((uint32_t)src * (uint32_t)p.ldx + (uint32_t)g * 128u) * 2u;
    const bool xrow = r16 < mrows;  // token lanes past the pass's rows read zeros, fetch nothing

    f32x4 acc2[RB], acc3[RB], acc4[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      acc2[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc3[rb] = acc2[rb];
      acc4[rb] = acc2[rb];
    }

    struct Set {
      uint32_t q[RB][2];
      uint32_t p3[RB], p4[RB];
      u32x4 x[4];
    };
    auto load = [&](Set& S, int st) __attribute__((always_inline)) {
      const int it = st >> 2, u = st & 3;
      const int itg = w * ipw + it;
      const bool live = st < nsub && itg < NI;  // uniform
      const uint32_t kq = (uint32_t)(itg * 512 + u * 32);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bool m0 = rb * 16 < RM;
        const uint32_t qo = live ? qoff[rb] + kq / 4 : qstrip;
        const auto qv = __builtin_amdgcn_raw_buffer_load_b64(m0 ? rq0 : rq1, (int)qo, 0, 0);
        S.q[rb][0] = qv[0];
        S.q[rb][1] = qv[1];
        const uint32_t po = live ? poff[rb] + kq / 8 : pstrip;
        if constexpr ((WM & 6) != 0)
          S.p3[rb] = __builtin_amdgcn_raw_buffer_load_b32(m0 ? r30 : r31, (int)po, 0, 0);
        else
          S.p3[rb] = 0u;
        if constexpr ((WM & 4) != 0)
          S.p4[rb] = __builtin_amdgcn_raw_buffer_load_b32(m0 ? r40 : r41, (int)po, 0, 0);
        else
          S.p4[rb] = 0u;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
        S.x[s] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       xres, (int)(live && xrow ? xoff + (kq + (uint32_t)s * 8u) * 2u : p.xbytes), 0, 0));
      // sets are issued whole and in order, so the oldest set is complete once
      // vmcnt <= the loads of the younger set
      __builtin_amdgcn_sched_barrier(0);
    };

    Tab tab[RB];
    auto tables = [&](int it) __attribute__((always_inline)) {
      // past the K range the tokens are zeros; any group's tables will do
      const int grp = min((w * ipw + it) * 4 + g, G - 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) build_tab<WM>(tab[rb], md[(rb * 16 + r16) * GP + grp]);
    };

    // MFMA step s of a sub-step covers the lane's weights 8s..8s+7: the quartets
    // (h, m) = (s / 2, 2 (s % 2)) and (s / 2, 2 (s % 2) + 1); each step's operands
    // are built right before its MFMAs, which keeps few of them live
    auto compute = [&](const Set& S) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 xb = as_bf16x8(S.x[s]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const Tab& T = tab[rb];
          u32x4 A2, A3, A4;
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const int h = s >> 1, m = 2 * (s & 1) + mm, d0 = 2 * mm;
            // bytes of t: 2-bit codes of the weights 16h + 4m + (0..3) of the sub-step
            const uint32_t t = (S.q[rb][h] >> (2 * m)) & 0x03030303u;
            const int i = 4 * h + m;           // their residual bits: bit 8b + i
            if constexpr ((WM & 1) != 0) {
              const uint32_t L = perm(0u, T.l2, t), H = perm(0u, T.h2, t);
              A2[d0] = pair01(L, H);
              A2[d0 + 1] = pair23(L, H);
            }
            if constexpr ((WM & 6) != 0) {
              const uint32_t c3 = t | (((S.p3[rb] >> i) & 0x01010101u) << 2);
              if constexpr ((WM & 2) != 0) {
                const uint32_t L = perm(T.l3[1], T.l3[0], c3), H = perm(T.h3[1], T.h3[0], c3);
                A3[d0] = pair01(L, H);
                A3[d0 + 1] = pair23(L, H);
              }
              if constexpr ((WM & 4) != 0) {
                // 0xff in the bytes whose r4 is set: byte 4 (of 0xffffffff) or byte 0 (of 0)
                const uint32_t m4 = perm(0xffffffffu, 0u, ((S.p4[rb] >> i) & 0x01010101u) << 2);
                const uint32_t L = (m4 & perm(T.l4[3], T.l4[2], c3)) |
                                   (~m4 & perm(T.l4[1], T.l4[0], c3));
                const uint32_t H = (m4 & perm(T.h4[3], T.h4[2], c3)) |
                                   (~m4 & perm(T.h4[1], T.h4[0], c3));
                A4[d0] = pair01(L, H);
                A4[d0 + 1] = pair23(L, H);
              }
            }
          }
          if constexpr ((WM & 1) != 0) acc2[rb] = mfma16(as_bf16x8(A2), xb, acc2[rb]);
          if constexpr ((WM & 2) != 0) acc3[rb] = mfma16(as_bf16x8(A3), xb, acc3[rb]);
          if constexpr ((WM & 4) != 0) acc4[rb] = mfma16(as_bf16x8(A4), xb, acc4[rb]);
        }
      }
    };

    Set st[2];
    load(st[0], 0);
    load(st[1], 1);
    if (mbase == 0) {
      // the first pass stages the metadata while its first operands are in flight
      stage_md();
      __syncthreads();
    }
    for (int it = 0; it < ipw; ++it) {
      tables(it);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        compute(st[u & 1]);
        load(st[u & 1], it * 4 + u + 2);
        // keep the next sub-step's MFMAs (and their waits) below this refill
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // each lane's token column takes the accumulator of its row's width
    const int mrel = mbase + r16;
    const int wid = mrel < b3 ? 2 : (mrel < b4 ? 3 : 4);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr ((WM & 1) != 0) a = (wid == 2) ? acc2[rb] : a;
      if constexpr ((WM & 2) != 0) a = (wid == 3) ? acc3[rb] : a;
      if constexpr ((WM & 4) != 0) a = (wid == 4) ? acc4[rb] : a;
      *(f32x4*)(red + (((w * RB) + rb) * 64 + lane) * 4) = a;
    }
    __syncthreads();
    for (int o = tid; o < 16 * NOUT; o += 256) {
      const int m = o / NOUT, col = o % NOUT;
      const int row = mbase + m;
      if (row >= cnt) continue;
      // C layout of the 16x16 MFMA: weight row 4*(lane/16)+i, token column lane%16
      auto part = [&](int wr) {
        const int rb = wr >> 4, rr = wr & 15;
        const int ln = (rr >> 2) * 16 + m, i = rr & 3;
        float sacc = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) sacc += red[((ww * RB + rb) * 64 + ln) * 4 + i];
        return sacc;
      };
      const size_t orow = (size_t)(row0 + row);
      if constexpr (MODE == kMModeGateUp) {
        const float gv = part(col), uv = part(RM + col);
        p.H[orow * p.N + n0 + col] = f32_to_bf16(silu_f32(gv) * uv);
      } else if constexpr (MODE == kMModeRelu) {
        p.H[orow * p.N + n0 + col] = f32_to_bf16(fmaxf(part(col), 0.0f));
      } else if constexpr (MODE == kMModeUp) {
        const float u = part(col);
        p.U[orow * p.N + n0 + col] = u;
        if (fabsf(u) > p.thr[e]) uflag[col] = 1;
      } else {
        const float gs = p.gate ? p.gate[p.gate_map[orow]] : 1.0f;
        p.Y[orow * p.N + n0 + col] = gs * part(col);
      }
    }
    __syncthreads();
  };

  if constexpr (MODE == kMModeUp) {
    for (int mbase = 0; mbase < cnt; mbase += 16) pass(std::integral_constant<int, 1>{}, mbase);
    __syncthreads();
    if (tid < RM) p.flags[(size_t)e * p.N + n0 + tid] = (uint8_t)uflag[tid];
    return;
  }
  for (int mbase = 0; mbase < cnt; mbase += 16) {
    const int hi = min(mbase + 16, cnt);
    const int wm = (mbase < b3 ? 1 : 0) | ((mbase < b4 && hi > b3) ? 2 : 0) | (hi > b4 ? 4 : 0);
    switch (wm) {
      case 1: pass(std::integral_constant<int, 1>{}, mbase); break;
      case 2: pass(std::integral_constant<int, 2>{}, mbase); break;
      case 3: pass(std::integral_constant<int, 3>{}, mbase); break;
      case 4: pass(std::integral_constant<int, 4>{}, mbase); break;
      case 5: pass(std::integral_constant<int, 5>{}, mbase); break;
      case 6: pass(std::integral_constant<int, 6>{}, mbase); break;
      default: pass(std::integral_constant<int, 7>{}, mbase); break;
    }
  }
}

template <int MODE, int RM>
size_t mwq_lds_bytes(int K) {
  constexpr int R = (MODE == kMModeGateUp) ? 2 * RM : RM;
  return (size_t)4 * (R / 16) * 64 * 16 + (size_t)R * ((K >> 7) + 1) * 8;
}

constexpr size_t kMwqMaxLds = 64 * 1024;
constexpr int kRmGateUp = MWQ_RM_GU, kRmDown = MWQ_RM_DN;

// rows: routed rows of the call, so at most min(E, rows) experts have any
template <int MODE, int RM>
hipError_t launch_mwq_mode(MwqArgs a, int E, int rows, hipStream_t s) {
  const size_t lds = mwq_lds_bytes<MODE, RM>(a.K);
  if (lds > kMwqMaxLds || E > kMaxExperts) return hipErrorInvalidValue;
  a.nblk_per_expert = a.N / RM;
  a.E = E;
  const int eact = rows < E ? rows : E;
  if (eact <= 0) return hipSuccess;
  hipLaunchKernelGGL((mwq_stream_kernel<MODE, RM>), dim3((unsigned)(eact * a.nblk_per_expert)),
                     dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace

const char* mwq_ffn_unsupported(int T, int d, int F, int k) {
  if (d % 512 != 0 || F % 512 != 0) return "nested experts need d_model and d_ff multiples of 512";
  if ((long long)T * d * 2 >= (1ll << 31) || (long long)T * k * F * 2 >= (1ll << 31))
    return "nested experts: token or hidden matrix too large for 32-bit offsets";
  if (mwq_lds_bytes<kMModeGateUp, kRmGateUp>(d) > kMwqMaxLds ||
      mwq_lds_bytes<kMModeDown, kRmDown>(F) > kMwqMaxLds)
    return "nested experts: d_model or d_ff too large for the group metadata in LDS";
  return nullptr;
}

hipError_t launch_mwq_ffn(const MwqProblem& p, hipStream_t s, hipEvent_t mid) {
  if (mwq_ffn_unsupported(p.T, p.d, p.F, p.k)) return hipErrorInvalidValue;
  const bool relu = p.act == MOE_ACT_RELU;
  MwqArgs a{};
  a.X = (const u16*)p.x;
  a.ldx = p.d;
  a.gather = p.row_assign;
  a.k = p.k;
  a.W0 = relu ? *p.w->up : *p.w->gate;
  a.W1 = *p.w->up;
  a.N = p.F;
  a.K = p.d;
  a.offsets = p.offsets;
  a.gpe = 3;
  a.H = (u16*)p.H;
  a.xbytes = (uint32_t)((size_t)p.T * p.d * 2);
  hipError_t e = relu ? launch_mwq_mode<kMModeRelu, kRmGateUp>(a, p.E, p.rows, s)
                      : launch_mwq_mode<kMModeGateUp, kRmGateUp>(a, p.E, p.rows, s);
  if (e != hipSuccess) return e;
  if (mid) {
    e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
  }
  MwqArgs b{};
  b.X = (const u16*)p.H;
  b.ldx = p.F;
  b.gather = nullptr;
  b.k = p.k;
  b.W0 = *p.w->down;
  b.W1 = *p.w->down;
  b.N = p.d;
  b.K = p.F;
  b.offsets = p.offsets;
  b.gpe = 3;
  b.Y = p.y_rows;
  b.gate_map = p.row_assign;
  b.gate = p.gate;
  b.xbytes = (uint32_t)((size_t)p.rows * p.F * 2);
  return launch_mwq_mode<kMModeDown, kRmDown>(b, p.E, p.rows, s);
}

hipError_t launch_int2_up(const void* x, int T, int d, int F, int E, int k, const moe_wmwq* w,
                          const int32_t* offsets, const int32_t* row_assign, const float* thr,
                          float* U, uint8_t* flags, hipStream_t s) {
  if (mwq_ffn_unsupported(T, d, F, k)) return hipErrorInvalidValue;
  MwqArgs a{};
  a.X = (const u16*)x;
  a.ldx = d;
  a.gather = row_assign;
  a.k = k;
  a.W0 = *w;
  a.W1 = *w;
  a.N = F;
  a.K = d;
  a.offsets = offsets;
  a.gpe = 1;
  a.U = U;
  a.thr = thr;
  a.flags = flags;
  a.xbytes = (uint32_t)((size_t)T * d * 2);
  // 64-column strips where their group metadata fits the LDS (faster at 16
  // tokens), else the down pass's 32
  if (mwq_lds_bytes<kMModeUp, 64>(d) <= kMwqMaxLds)
    return launch_mwq_mode<kMModeUp, 64>(a, E, T * k, s);
  return launch_mwq_mode<kMModeUp, kRmDown>(a, E, T * k, s);
}

}  // namespace moe
