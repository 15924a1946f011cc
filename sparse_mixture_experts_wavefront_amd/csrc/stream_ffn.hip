// stream_ffn.hip -- grouped expert FFN for few rows per expert (decode).
//
// With a handful of token rows per expert the FFN is a weight stream: every
// weight byte is read once and each feeds only a few multiply-adds, so HBM
// bandwidth bounds it ("FloE: On-the-Fly MoE Inference on Memory-constrained
// GPU" -- What carries the argument: decode time goes to moving expert weights;
// "D^2MoE: Dual Routing and Dynamic Scheduling for Efficient On-Device
// MoE-based LLM Serving" -- What carries the argument and Figure 8: low-bit
// expert weights are decoded inside the GEMM kernel).
//
// One block = one expert x one strip of output columns (64 weight rows for
// gate/up: 32 gate + 32 up, the same f-values; for ReLU W_in and for down 32
// rows; twice those in the register-direct INT4 kernel); its 4 waves split K and their partial sums meet in LDS at the end,
// where the epilogue applies SiLU(gate)*up (to bf16 H) or the gate scale (fp32
// rows).  Two ways to feed the 16x16x32 MFMA from the weight stream:
//   register-direct (gate/up, ReLU W_in, INT4 down): each wave loads its MFMA
//     operands straight into registers, 16 row pieces of 64 bytes per
//     instruction, with ordinary cached loads (the other half of each 128-byte
//     line is the next instruction's piece and hits L2; measured ~12% faster
//     than non-temporal loads for this pattern on MI355X);
//   LDS-staged (bf16 down, K = d_ff long rows): non-temporal 16-byte loads laid
//     out so one wave instruction reads whole 1 KB row pieces (~7 TB/s from HBM
//     for this pattern, ~5-5.6 TB/s for the MFMA-shaped one, ~5.5 TB/s through
//     LDS DMA), written to one of two LDS slots in the MFMA operand layout.
// LDS-staged details: weights stream in chunks of 512 K values (bf16: 16 rows x
// 1 KB; INT4: all rows x 256 B), loaded two chunks ahead into registers, stored
// to the slot, published by a barrier and multiplied by the 4 waves, each taking
// a quarter of the chunk's K range, against the expert's token rows (up to 16
// per B operand, zero-padded).
//
// INT4 weights (group 128 along K, fp16 scale s and zero z, 8 nibbles per
// int32, low nibble first) are decoded in registers right before the MFMA:
//   W = bf16_RNE( fp32( fp32(q) - z ) * s )
// When fp32(q) - z is exact for every q in 0..15 (z == 0 or |z| >= 2^-10), this
// equals bf16_RNE( fma(q, s, -(z*s)) ): z*s is exact in fp32 (11+11 bits) and
// the fma rounds the exact (q - z)*s once.  The fused form is used only where
// every zero point involved allows it (per chunk in the LDS-staged kernel, per
// block in the register-direct one), the two-operation form otherwise.
// LDS-staged K map: within a chunk, lane (r, g) of wave w feeds MFMA step s with K values
// [w*128 + g*32 + s*8, +8); the token operand uses the same map, so the MFMA
// sums over the same K set (the order of K inside one accumulation is free).
// LDS rows keep 16-byte unit u of row r at position u ^ (r & 15), so the 16 rows
// one read pass touches fall on 16 different bank groups.
#include <mutex>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSModeGateUp = 0, kSModeRelu = 1, kSModeDown = 2;


struct StreamArgs {
  const u16* X;            // gate/up: x [T][ldx]; down: H [rows][ldx]
  int ldx;
  const int32_t* gather;   // gate/up: row -> flat assignment (token = a / k); NULL: row
  int k;
  const unsigned char* W0; // dense bf16 or INT4 words, [E][N][K] elements
  const unsigned char* W1;
  const u16* s0; const u16* s1; const u16* z0; const u16* z1;   // INT4 fp16 [E][N][K/128]
  int N, K;
  const int32_t* offsets;  // [E+1] or NULL (one expert, `rows` rows)
  int rows;
  u16* H;                  // gate/up output [rows][N]
  float* Y;                // down output [rows][N]
  float* Yacc;             // down: if not NULL, row r is added into Yacc[gate_map[r] / k][N]
  const int32_t* gate_map;
  const float* gate;
  int nblk_per_expert;
  uint32_t xbytes;         // bytes of X (register-direct kernel: buffer size)
  int sz_vec;              // INT4: scales / zero points 16-byte aligned, K % 1024 == 0 and
                           // R*K/1024 <= 2048: staged with 16-byte loads
  f32x4* zero;             // gate/up: if not NULL, the grid zeroes zero[0 .. zero_n4) first
  size_t zero_n4;          // (the output the down pass then accumulates into)
  int kparts;              // row-split down: K parts; part q writes its partial rows
  size_t ystride;          // to Y + q * ystride (summed by the combine)
};

// the whole grid zeroes p.zero (spread over all blocks, before any exits)
__device__ __forceinline__ void grid_zero(const StreamArgs& p) {
  if (!p.zero) return;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < p.zero_n4;
       i += (size_t)gridDim.x * blockDim.x)
    p.zero[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// fp32(q) - z is exact for all q in 0..15 when z == 0 or |z| >= 2^-10 (finite).
__device__ __forceinline__ bool zero_point_fma_exact(u16 z) {
  const unsigned ex = (z >> 10) & 0x1f;
  return (z & 0x7fff) == 0 || (ex >= 5 && ex != 31);
}

// byte b of v as fp32 (v_cvt_f32_ubyte{b}; plain VALU, no memory access)
__device__ __forceinline__ float ub0(uint32_t v) { float f; asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(v)); return f; }
__device__ __forceinline__ float ub1(uint32_t v) { float f; asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(v)); return f; }
__device__ __forceinline__ float ub2(uint32_t v) { float f; asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(v)); return f; }
__device__ __forceinline__ float ub3(uint32_t v) { float f; asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(v)); return f; }

// 8 nibbles (low first) -> 8 bf16, fused form: fma(q, s, nzs), nzs = -(z*s) exact.
__device__ __forceinline__ bf16x8 dq8_fma(uint32_t w, float s, float nzs) {
  const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;  // nibbles 0,2,4,6 / 1,3,5,7
  u32x4 o;
  o[0] = pk_bf16(__builtin_fmaf(ub0(lo), s, nzs), __builtin_fmaf(ub0(hi), s, nzs));
  o[1] = pk_bf16(__builtin_fmaf(ub1(lo), s, nzs), __builtin_fmaf(ub1(hi), s, nzs));
  o[2] = pk_bf16(__builtin_fmaf(ub2(lo), s, nzs), __builtin_fmaf(ub2(hi), s, nzs));
  o[3] = pk_bf16(__builtin_fmaf(ub3(lo), s, nzs), __builtin_fmaf(ub3(hi), s, nzs));
  return as_bf16x8(o);
}
// The same fused decode with the int-to-float conversion folded into the fma:
// a 16-bit half that holds a nibble q in bits 0-3 (or 4-7) and zeros elsewhere
// is the fp16 subnormal q * 2^-24 (q * 2^-20), which v_fma_mix_f32 reads as an
// exact fp32 operand; with the scale pre-multiplied by 2^24 (2^20), also exact,
// fma(q * 2^-24, s * 2^24, nzs) is fma(q, s, nzs) rounded once.  Four masks and
// one shift place all 8 nibbles (fp16 denormals are kept: the kernels run with
// the default denormal mode).
__device__ __forceinline__ float mix_lo(uint32_t m, float s, float c) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(m), "v"(s), "v"(c));
  return r;
}
__device__ __forceinline__ float mix_hi(uint32_t m, float s, float c) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(m), "v"(s), "v"(c));
  return r;
}
__device__ __forceinline__ bf16x8 dq8_mix(uint32_t w, float s, float nzs) {
  const float s24 = s * 16777216.0f, s20 = s * 1048576.0f;
  const uint32_t w8 = w >> 8;
  const uint32_t m0 = w & 0x000f000fu, m1 = w & 0x00f000f0u;    // nibbles 0, 4 / 1, 5
  const uint32_t m2 = w8 & 0x000f000fu, m3 = w8 & 0x00f000f0u;  // nibbles 2, 6 / 3, 7
  u32x4 o;
  o[0] = pk_bf16(mix_lo(m0, s24, nzs), mix_lo(m1, s20, nzs));
  o[1] = pk_bf16(mix_lo(m2, s24, nzs), mix_lo(m3, s20, nzs));
  o[2] = pk_bf16(mix_hi(m0, s24, nzs), mix_hi(m1, s20, nzs));
  o[3] = pk_bf16(mix_hi(m2, s24, nzs), mix_hi(m3, s20, nzs));
  return as_bf16x8(o);
}
// the defining two-operation form (any zero point)
__device__ __forceinline__ bf16x8 dq8_exact(uint32_t w, float s, float z) {
  const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
  auto f = [&](float q) { return __fmul_rn(__fsub_rn(q, z), s); };
  u32x4 o;
  o[0] = pk_bf16(f(ub0(lo)), f(ub0(hi)));
  o[1] = pk_bf16(f(ub1(lo)), f(ub1(hi)));
  o[2] = pk_bf16(f(ub2(lo)), f(ub2(hi)));
  o[3] = pk_bf16(f(ub3(lo)), f(ub3(hi)));
  return as_bf16x8(o);
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int gcd_c(int a, int b) { return b ? gcd_c(b, a % b) : a; }
constexpr int lcm3(int a, int b, int c) {
  const int ab = a / gcd_c(a, b) * b;
  return ab / gcd_c(ab, c) * c;
}

template <int MODE, bool INT4, int MB>
__global__ __launch_bounds__(256) void stream_ffn_kernel(StreamArgs p) {
  constexpr int R = (MODE == kSModeGateUp) ? 64 : 32;  // weight rows per block
  constexpr int RBLK = R / 16;
  constexpr int NOUT = 32;                              // output columns per block
  constexpr int KC = 512, KW = 128, NS = 4, KL = 32;    // K per chunk / wave / MFMA steps / lane
  constexpr int CR = INT4 ? R : 16;                     // weight rows per chunk
  constexpr int RBYTES = INT4 ? KC / 2 : KC * 2;        // bytes per row per chunk (256 | 1024)
  constexpr int CBYTES = CR * RBYTES;                   // 16 KB (8 KB for INT4 ReLU/down)
  constexpr int NRC = R / CR;                           // chunks per K slice
  constexpr int CRB = CR / 16;                          // 16-row blocks per chunk
  constexpr int UPR = RBYTES / 16;                      // 16-byte units per row per chunk
  constexpr int NLD = CBYTES / 1024 / 4;                // 16-byte weight loads per lane per chunk
  constexpr int WU = INT4 ? 1 : 4;                      // 16-byte units per lane per row block
  constexpr int D = (INT4 && MB > 1) ? 1 : 2;           // chunks loaded ahead
  constexpr int NSET = D + 1;
  // unroll: a common multiple of the register sets, the 2 LDS slots and the
  // chunks per K slice, so set, slot and row block are compile-time in the body
  constexpr int U = lcm3(NSET, 2, NRC);
  static_assert(UPR >= 16 && NLD >= 1, "geometry");

  __shared__ __align__(16) unsigned char sW0[CBYTES], sW1[CBYTES];

  grid_zero(p);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = blockIdx.x / p.nblk_per_expert;
  const int nb = blockIdx.x - e * p.nblk_per_expert;
  int row0 = 0, cnt = p.rows;
  if (p.offsets) {
    row0 = p.offsets[e];
    cnt = p.offsets[e + 1] - row0;
  }
  row0 = __builtin_amdgcn_readfirstlane(row0);
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  if (cnt <= 0) return;
  const int n0 = nb * NOUT;
  const int r16 = lane & 15, g = lane >> 4;
  const int nchunks = (p.K / KC) * NRC;
  const int kgroups = p.K >> 7;
  const size_t row_bytes = INT4 ? (size_t)p.K / 2 : (size_t)p.K * 2;

  // block row r (0..R-1) -> weight matrix and row
  auto wsel = [&](int r, const unsigned char*& W, int& n) {
    if constexpr (MODE == kSModeGateUp) {
      W = (r < 32) ? p.W0 : p.W1;
      n = n0 + (r & 31);
    } else {
      W = p.W0;
      n = n0 + r;
    }
    n = min(n, p.N - 1);
  };
  // Loads: load j of wave w covers chunk units (w*NLD+j)*64 + lane, i.e. chunk
  // row u / UPR, unit u % UPR: one wave instruction reads RBYTES-long contiguous
  // row pieces (1 KB for bf16).  N is a multiple of the strip width (checked by
  // the launcher), so a chunk's rows are a fixed offset from chunk 0's rows.
  const unsigned char* lsrc[NLD];
  const unsigned char* lsrc_up[NLD];
  int ldst[NLD];  // LDS byte offset of the unit (chunk row r, unit pos ^ (r & 15))
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int u = (w * NLD + j) * 64 + lane;
    const int r = u / UPR, pos = u % UPR;
    const unsigned char* W;
    int n;
    wsel(r, W, n);
    lsrc[j] = W + ((size_t)e * p.N + n) * row_bytes + pos * 16;
    if constexpr (MODE == kSModeGateUp && NRC > 1) {
      wsel(32 + r, W, n);
      lsrc_up[j] = W + ((size_t)e * p.N + n) * row_bytes + pos * 16;
    } else {
      lsrc_up[j] = lsrc[j];
    }
    ldst[j] = r * RBYTES + ((pos ^ (r & 15)) * 16);
  }

  const u16* sz_s[RBLK];
  const u16* sz_z[RBLK];
  if constexpr (INT4) {
#pragma unroll
    for (int rb = 0; rb < RBLK; ++rb) {
      const int r = rb * 16 + r16;
      const unsigned char* W;
      int n;
      wsel(r, W, n);
      const bool second = (MODE == kSModeGateUp) && r >= 32;
      sz_s[rb] = (second ? p.s1 : p.s0) + ((size_t)e * p.N + n) * kgroups;
      sz_z[rb] = (second ? p.z1 : p.z0) + ((size_t)e * p.N + n) * kgroups;
    }
  }

  __shared__ float gsm[MB * 16];  // down: gates of this pass's token rows
  for (int mbase = 0; mbase < cnt; mbase += MB * 16) {
    const int mrows = min(MB * 16, cnt - mbase);
    const int mb_act = (mrows + 15) >> 4;
    // down: the gate of row tid of this pass, loaded before the weight stream
    float gpre = 1.0f;
    if constexpr (MODE == kSModeDown) {
      if (p.gate && tid < MB * 16) {
        const int rr = row0 + mbase + min(tid, mrows - 1);
        gpre = p.gate[p.gate_map ? p.gate_map[rr] : rr];
      }
    }
    const u16* xrow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + r16;
      const int rr = row0 + mbase + min(m, mrows - 1);
      const int src = p.gather ? p.gather[rr] / p.k : rr;
      xrow[mb] = p.X + (size_t)src * p.ldx + w * KW + g * KL;
    }
    f32x4 acc[RBLK][MB];
#pragma unroll
    for (int rb = 0; rb < RBLK; ++rb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    struct Set {
      u32x4 wv[NLD];
      u32x4 x[MB][NS];
      u16 s[CRB], z[CRB];
    };
    // chunk c = (kc, rc): rows rc*CR.., K [kc*KC, +KC); lane (r, g) feeds MFMA
    // step s with K [w*KW + g*KL + s*8, +8) of it (weights and tokens alike)
    auto load = [&](Set& st, int c) {
      const int kc = c / NRC, rc = c - kc * NRC;
      const bool up = (MODE == kSModeGateUp && NRC > 1) && rc >= NRC / 2;
      const size_t roff = (size_t)kc * RBYTES + (size_t)((NRC > 1 ? rc : 0) & 1) * 16 * row_bytes;
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        st.wv[j] = __builtin_nontemporal_load((const u32x4*)((up ? lsrc_up[j] : lsrc[j]) + roff));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)  // rows past the count are clamped copies
#pragma unroll
        for (int s = 0; s < NS; ++s) st.x[mb][s] = *(const u32x4*)(xrow[mb] + (size_t)kc * KC + s * 8);
      if constexpr (INT4) {
        const int grp = (kc * KC + w * KW + g * KL) >> 7;
#pragma unroll
        for (int i = 0; i < CRB; ++i) {
          st.s[i] = sz_s[rc * CRB + i][grp];
          st.z[i] = sz_z[rc * CRB + i][grp];
        }
      }
    };
    auto store = [&](unsigned char* slot, const Set& st) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) *(u32x4*)(slot + ldst[j]) = st.wv[j];
    };
    auto compute = [&](const unsigned char* slot, const Set& st, int rc) {
      const int ubase = INT4 ? (w * KW + g * KL) / 32 : (w * KW + g * KL) / 8;
      u32x4 wv[CRB][WU];
#pragma unroll
      for (int i = 0; i < CRB; ++i) {
        const int r = i * 16 + r16;
#pragma unroll
        for (int q = 0; q < WU; ++q)
          wv[i][q] = *(const u32x4*)(slot + r * RBYTES + (((ubase + q) ^ (r & 15)) * 16));
      }
      if constexpr (!INT4) {
#pragma unroll
        for (int i = 0; i < CRB; ++i)
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[rc * CRB + i][mb] = mfma16(as_bf16x8(wv[i][s]), as_bf16x8(st.x[mb][s]),
                                             acc[rc * CRB + i][mb]);
      } else {
        float sf[CRB], zf[CRB], nzs[CRB];
        bool ok = true;
#pragma unroll
        for (int i = 0; i < CRB; ++i) {
          sf[i] = h2f(st.s[i]);
          zf[i] = h2f(st.z[i]);
          nzs[i] = -(zf[i] * sf[i]);
          ok = ok && zero_point_fma_exact(st.z[i]);
        }
        // one uniform choice per chunk: the fused decode when every zero point
        // of the chunk allows it (the usual case), else the two-operation form
        const bool fast =
            __builtin_amdgcn_readfirstlane((int)(__ballot(!ok) == 0ull)) != 0;
        auto run = [&](auto fused) {
#pragma unroll
          for (int i = 0; i < CRB; ++i) {
            bf16x8 a[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              if constexpr (decltype(fused)::value)
                a[s] = dq8_fma(wv[i][0][s], sf[i], nzs[i]);
              else
                a[s] = dq8_exact(wv[i][0][s], sf[i], zf[i]);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int mb = 0; mb < MB; ++mb)
                acc[rc * CRB + i][mb] = mfma16(a[s], as_bf16x8(st.x[mb][s]), acc[rc * CRB + i][mb]);
          }
        };
        if (fast)
          run(std::true_type{});
        else
          run(std::false_type{});
      }
    };

    // ---- pipeline: chunk c sits in register set c % NSET (loaded D chunks
    // ahead), goes to LDS slot c % 2, is published by the barrier and multiplied.
    // Slot c % 2 was last read in iteration c - 2, which every wave finished
    // before the barrier of iteration c - 1.
    Set st[NSET];
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < nchunks) load(st[d], d);
    for (int c0 = 0; c0 < nchunks; c0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u;
        if (c < nchunks) {  // uniform
          unsigned char* slot = (u & 1) ? sW1 : sW0;
          store(slot, st[u % NSET]);
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
          block_barrier();
          if (c + D < nchunks) load(st[(u + D) % NSET], c + D);
          compute(slot, st[u % NSET], u % NRC);  // c0 is a multiple of U, so rc = u % NRC
        }
      }
    }

    // ---- cross-wave reduction and epilogue, one 16-row token block at a time ----
    float* red = (float*)sW0;  // [4 waves][RBLK][64 lanes][4]
    static_assert(4 * RBLK * 64 * 16 <= CBYTES, "reduction buffer");
    if (tid < MB * 16) gsm[tid] = gpre;  // published by the barrier below
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= mb_act) break;
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < RBLK; ++rb)
        *(f32x4*)(red + (((w * RBLK) + rb) * 64 + lane) * 4) = acc[rb][mb];
      __syncthreads();
      for (int o = tid; o < 16 * NOUT; o += 256) {
        const int m = o / NOUT, col = o % NOUT;
        const int row = mbase + mb * 16 + m;
        if (row >= cnt || n0 + col >= p.N) continue;
        // C layout of 16x16 MFMA: weight row 4*(lane/16)+i, token column lane%16
        auto part = [&](int wr) {
          const int rb = wr >> 4, rr = wr & 15;
          const int ln = (rr >> 2) * 16 + m, i = rr & 3;
          float sacc = 0.0f;
#pragma unroll
          for (int ww = 0; ww < 4; ++ww) sacc += red[((ww * RBLK + rb) * 64 + ln) * 4 + i];
          return sacc;
        };
        const size_t orow = (size_t)(row0 + row);
        if constexpr (MODE == kSModeGateUp) {
          const float gv = part(col), uv = part(32 + col);
          p.H[orow * p.N + n0 + col] = f32_to_bf16(silu_f32(gv) * uv);
        } else if constexpr (MODE == kSModeRelu) {
          p.H[orow * p.N + n0 + col] = f32_to_bf16(fmaxf(part(col), 0.0f));
        } else {
          const float v = gsm[mb * 16 + m] * part(col);
          if (p.Yacc)
            unsafeAtomicAdd(p.Yacc + (size_t)(p.gate_map[orow] / p.k) * p.N + n0 + col, v);
          else
            p.Y[orow * p.N + n0 + col] = v;
        }
      }
    }
    __syncthreads();
  }
}

// ---- register-direct variant ------------------------------------------------
// Each wave owns a contiguous quarter of K for all of the block's weight rows
// and loads its MFMA operands straight into registers (lane (r, g) of a wave
// instruction reads 16 bytes of weight row r; the 4 lanes of a row are
// adjacent, so one instruction reads 16 row pieces of 64 bytes), D iterations
// ahead, with no LDS staging and no barrier until the final K reduction.
// Iteration = 128 K values = one INT4 group.  K map inside an iteration, the
// same for weights and tokens: bf16 lane (r, g) step s takes K [s*32 + g*8, +8);
// INT4 lane (r, g) holds K [g*32, +32) in one 16-byte load and feeds step s
// with its word s, i.e. K [g*32 + s*8, +8).  INT4 scales and zero points of the
// block's rows are staged once in LDS (row stride G+1 words: 16 rows hit 16
// different banks).
// The loop has no data-dependent branch: loads run through buffer resources,
// and an iteration past the wave's K range loads from an offset past the
// resource's size, which returns zeros without touching memory; its MFMAs then
// add zeros.  A straight-line loop lets the compiler wait for exactly the
// oldest register set (vmcnt = loads of the D-1 younger sets) instead of all.

constexpr int stream_reg_rows(int mode, bool int4) {
  return mode == kSModeGateUp ? (int4 ? 128 : 64) : (int4 ? 64 : 32);
}

template <int MODE, bool INT4, int MB, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(INT4 ? 2 : 1)))
void stream_reg_kernel(StreamArgs p) {
  // weight rows per block: gate/up 32 gate + 32 up rows (INT4: 64 + 64); down
  // and ReLU W_in 32 rows (INT4: 64).  More rows let each token fragment feed
  // more MFMAs, fewer token-operand loads per weight byte; the INT4 weight
  // registers leave room for that
  constexpr int R = stream_reg_rows(MODE, INT4);
  constexpr int RB = R / 16;
  constexpr int NOUT = (MODE == kSModeGateUp) ? R / 2 : R;
  constexpr int SR = (MODE == kSModeGateUp) ? R / 2 : 32;  // weight rows per buffer resource
  constexpr int KI = 128, NS = 4;
  constexpr int WL = INT4 ? 1 : NS;                  // 16-byte weight loads per row block
  constexpr int IT_BYTES = INT4 ? KI / 2 : KI * 2;    // weight bytes per row per iteration
  constexpr int XS = INT4 ? 8 : 32;                  // token K offset between MFMA steps

  extern __shared__ __align__(16) unsigned char smem[];
  float* red = (float*)smem;                                 // [4][RB][64][4]
  uint32_t* sz = (uint32_t*)(smem + 4 * RB * 64 * 16);       // [R][G+1]: s | z << 16

  grid_zero(p);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = blockIdx.x / p.nblk_per_expert;
  const int nb = blockIdx.x - e * p.nblk_per_expert;
  int row0 = 0, cnt = p.rows;
  if (p.offsets) {
    row0 = p.offsets[e];
    cnt = p.offsets[e + 1] - row0;
  }
  row0 = __builtin_amdgcn_readfirstlane(row0);
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  if (cnt <= 0) return;
  const int n0 = nb * NOUT;
  const int r16 = lane & 15, g = lane >> 4;
  const int Kq = p.K >> 2;            // per wave; a multiple of KI (K % 512 == 0)
  const int kw0 = w * Kq;
  const int iters = Kq / KI;
  const int G = p.K >> 7, GP = G + 1;
  const uint32_t row_bytes = INT4 ? (uint32_t)p.K / 2 : (uint32_t)p.K * 2;

  // weight resources: SR rows of the block's strip each (the launcher checks
  // that 64 rows and the token matrix fit 32-bit offsets)
  const uint32_t strip_bytes = (uint32_t)SR * row_bytes;
  const __amdgpu_buffer_rsrc_t wres0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.W0 + ((size_t)e * p.N + n0) * row_bytes), (short)0, (int)strip_bytes, 0x00020000);
  // (gate/up: the up matrix's strip; 64-row blocks: rows 32..63 of the block)
  const __amdgpu_buffer_rsrc_t wres1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(MODE == kSModeGateUp ? p.W1 + ((size_t)e * p.N + n0) * row_bytes
                                   : p.W0 + ((size_t)e * p.N + n0 + (R == 64 ? 32 : 0)) * row_bytes),
      (short)0, (int)strip_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.X, (short)0, (int)p.xbytes, 0x00020000);
  // row block rb covers block rows rb*16..+15: matrix 0 for rows < 32, 1 above
  uint32_t wvoff[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    wvoff[rb] = (uint32_t)((rb * 16 + r16) & (SR - 1)) * row_bytes +
                (INT4 ? (uint32_t)(kw0 + g * 32) / 2 : (uint32_t)(kw0 + g * 8) * 2);

  auto wsel = [&](int r, int& n, bool& second) {
    if constexpr (MODE == kSModeGateUp) {
      second = r >= SR;
      n = n0 + (r & (SR - 1));
    } else {
      second = false;
      n = n0 + r;
    }
  };
  bool fused_ok = true;
  if constexpr (INT4) {
    bool ok = true;
    if (p.sz_vec) {
      // 8 groups (16 bytes of scales, 16 of zero points) per load; a thread's
      // loads are issued together, so the staging costs one memory round trip
      const int G8 = G >> 3;
      constexpr int kMaxPer = 8;  // R * G / 8 / 256 <= 8 for K <= 16384
      u32x4 sv[kMaxPer], zv[kMaxPer];
#pragma unroll
      for (int q = 0; q < kMaxPer; ++q) {
        const int i = tid + q * 256;
        if (i < R * G8) {
          const int r = i / G8, j = i - r * G8;
          int n;
          bool second;
          wsel(r, n, second);
          const size_t o = ((size_t)e * p.N + n) * G + j * 8;
          sv[q] = *(const u32x4*)((second ? p.s1 : p.s0) + o);
          zv[q] = *(const u32x4*)((second ? p.z1 : p.z0) + o);
        }
      }
#pragma unroll
      for (int q = 0; q < kMaxPer; ++q) {
        const int i = tid + q * 256;
        if (i < R * G8) {
          const int r = i / G8, j = i - r * G8;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint32_t s2 = sv[q][h], z2 = zv[q][h];
            ok = ok && zero_point_fma_exact((u16)(z2 & 0xffffu)) && zero_point_fma_exact((u16)(z2 >> 16));
            sz[r * GP + j * 8 + 2 * h] = (s2 & 0xffffu) | (z2 << 16);
            sz[r * GP + j * 8 + 2 * h + 1] = (s2 >> 16) | (z2 & 0xffff0000u);
          }
        }
      }
    } else {
      for (int i = tid; i < R * G; i += 256) {
        const int r = i / G, gi = i - r * G;
        int n;
        bool second;
        wsel(r, n, second);
        const size_t o = ((size_t)e * p.N + n) * G + gi;
        const u16 s = (second ? p.s1 : p.s0)[o], z = (second ? p.z1 : p.z0)[o];
        ok = ok && zero_point_fma_exact(z);
        sz[r * GP + gi] = (uint32_t)s | ((uint32_t)z << 16);
      }
    }
    // the fused decode when every zero point of the block allows it (the usual
    // case), else the two-operation form; uniform over the block
    fused_ok = __syncthreads_and(ok) != 0;
  }

  __shared__ float gsm[MB * 16];  // down: gates of this pass's token rows
  auto body = [&](auto fused) {
    for (int mbase = 0; mbase < cnt; mbase += MB * 16) {
      const int mrows = min(MB * 16, cnt - mbase);
      const int mb_act = (mrows + 15) >> 4;
      // down: the gate of row tid of this pass, loaded before the weight stream
      float gpre = 1.0f;
      if constexpr (MODE == kSModeDown) {
        if (p.gate && tid < MB * 16) {
          const int rr = row0 + mbase + min(tid, mrows - 1);
          gpre = p.gate[p.gate_map ? p.gate_map[rr] : rr];
        }
      }
      uint32_t xvoff[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = mb * 16 + r16;
        const int rr = row0 + mbase + min(m, mrows - 1);  // rows past the count: clamped copies
        const int src = p.gather ? p.gather[rr] / p.k : rr;
        xvoff[mb] = ((uint32_t)src * (uint32_t)p.ldx + (uint32_t)(kw0 + (INT4 ? g * 32 : g * 8))) * 2u;
      }
      f32x4 acc[RB][MB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

      struct Set {
        u32x4 wv[RB][WL];
        u32x4 x[MB][NS];
      };
      auto load = [&](Set& S, int it) {
        const bool live = it < iters;  // uniform
        const uint32_t wo = live ? (uint32_t)it * IT_BYTES : strip_bytes;
        const uint32_t xo = live ? (uint32_t)it * KI * 2 : p.xbytes;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int q = 0; q < WL; ++q)
            S.wv[rb][q] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128((rb * 16 < SR) ? wres0 : wres1,
                                                             (int)(wvoff[rb] + wo + q * 64), 0, 0));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int s = 0; s < NS; ++s)
            S.x[mb][s] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, (int)(xvoff[mb] + xo + s * XS * 2),
                                                             0, 0));
        // sets are issued whole and in order (prologue and loop alike), so the
        // oldest set is complete once vmcnt <= the loads of the younger sets
        __builtin_amdgcn_sched_barrier(0);
      };
      auto compute = [&](const Set& S, int it) {
        if constexpr (!INT4) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int mb = 0; mb < MB; ++mb)
                acc[rb][mb] = mfma16(as_bf16x8(S.wv[rb][s]), as_bf16x8(S.x[mb][s]), acc[rb][mb]);
        } else {
          // past the K range the tokens are zeros; any finite scale will do
          const int grp = (kw0 >> 7) + min(it, iters - 1);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const uint32_t v = sz[(rb * 16 + r16) * GP + grp];
            const float sf = h2f((u16)(v & 0xffffu)), zf = h2f((u16)(v >> 16));
            const float nzs = -(zf * sf);
            bf16x8 a[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              if constexpr (decltype(fused)::value)
                a[s] = dq8_mix(S.wv[rb][0][s], sf, nzs);
              else
                a[s] = dq8_exact(S.wv[rb][0][s], sf, zf);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int mb = 0; mb < MB; ++mb)
                acc[rb][mb] = mfma16(a[s], as_bf16x8(S.x[mb][s]), acc[rb][mb]);
          }
        }
      };

      // iteration it lives in register set it % D, loaded D iterations ahead;
      // its set is refilled with iteration it + D once its MFMAs are issued
      Set st[D];
#pragma unroll
      for (int d = 0; d < D; ++d) load(st[d], d);
      for (int it0 = 0; it0 < iters; it0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
          compute(st[u], it0 + u);
          load(st[u], it0 + u + D);
          // keep the scheduler from hoisting the next set's MFMAs (and their
          // waits) above this set's refill
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // cross-wave K reduction and epilogue, one 16-row token block at a time
      if (tid < MB * 16) gsm[tid] = gpre;  // published by the barrier below
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (mb >= mb_act) break;
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          *(f32x4*)(red + (((w * RB) + rb) * 64 + lane) * 4) = acc[rb][mb];
        __syncthreads();
        for (int o = tid; o < 16 * NOUT; o += 256) {
          const int m = o / NOUT, col = o % NOUT;
          const int row = mbase + mb * 16 + m;
          if (row >= cnt || n0 + col >= p.N) continue;
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
          if constexpr (MODE == kSModeGateUp) {
            const float gv = part(col), uv = part(SR + col);
            p.H[orow * p.N + n0 + col] = f32_to_bf16(silu_f32(gv) * uv);
          } else if constexpr (MODE == kSModeRelu) {
            p.H[orow * p.N + n0 + col] = f32_to_bf16(fmaxf(part(col), 0.0f));
          } else {
            const float v = gsm[mb * 16 + m] * part(col);
            if (p.Yacc)
              unsafeAtomicAdd(p.Yacc + (size_t)(p.gate_map[orow] / p.k) * p.N + n0 + col, v);
            else
              p.Y[orow * p.N + n0 + col] = v;
          }
        }
      }
      __syncthreads();
    }
  };
  if constexpr (INT4) {
    if (fused_ok)
      body(std::true_type{});
    else
      body(std::false_type{});
  } else {
    body(std::true_type{});
  }
}

// ---- row-split variant (INT4 gate/up, ReLU W_in and down, few token rows) -----
// The K-split kernel above gives each wave a quarter of K for all of the
// block's rows, so each wave loads its own token fragments and a token byte
// feeds only the block's 64-128 rows.  Here each wave owns RBW 16-row blocks of
// weight rows (gate/up: RBW/2 blocks of gate rows and the matching up rows)
// over the whole of K and the four waves share the token fragments: each
// 128-K slice of the block's token rows is loaded once per block (one 16-byte
// load per thread and 16-row token block), stored to one of two LDS slots (row
// stride 272 bytes, so the 16 rows one MFMA operand read touches fall on 16
// different bank groups) and read by all four waves, one barrier per slice.  A
// block covers 4*RBW*16 weight rows of each matrix's strip for up to MB*16
// token rows per pass; no cross-wave reduction is needed, each wave applies
// the epilogue to its own accumulators.  Weights are loaded D slices ahead
// into registers, token slices one slice ahead.  K map inside a slice, INT4
// scale table and out-of-range loads as in the K-split kernel.  The down pass
// (N = d_model is short: strips alone would give too few blocks) also splits K
// into p.kparts parts, one block each; a block writes its gate-scaled partial
// rows to Y + part * ystride and the combine adds the parts in part order, so
// the result does not depend on block timing.
constexpr int kRowsRBW = 4;                      // 16-row weight blocks per wave (default)
// LDS bytes per staged token row of a slice of 128*WQ K values (16 bytes of padding)
constexpr int rows_xrow(int wq) { return 128 * wq * 2 + 16; }

template <int MODE, int RBW>
constexpr int stream_rows_nout() { return MODE == kSModeGateUp ? 4 * RBW * 8 : 4 * RBW * 16; }

template <int MODE, bool INT4, int MB, int D, int WQ, int RBW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void stream_rows_kernel(StreamArgs p) {
  static_assert(INT4 || WQ == 1, "bf16 slices are 128 K values");
  constexpr int KI = 128 * WQ, NS = 4;
  constexpr int WL = INT4 ? WQ : NS;                  // 16-byte weight loads per row block
  constexpr int IT_BYTES = INT4 ? KI / 2 : KI * 2;    // weight bytes per row per slice
  constexpr int NWF = (MODE == kSModeGateUp) ? RBW * 8 : RBW * 16;  // output columns per wave
  constexpr int NOUT = stream_rows_nout<MODE, RBW>(); // per block (= rows per weight strip)
  constexpr int XROW = rows_xrow(WQ);
  constexpr int XSLOT = MB * 16 * XROW;

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* xs = smem;                                  // [2][MB*16][XROW]
  uint32_t* sz = (uint32_t*)(smem + 2 * XSLOT);              // [4*RBW*16][G+1]: s | z << 16
  __shared__ float gsm[MB * 16];                             // down: gates of the pass's rows

  grid_zero(p);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = blockIdx.x / p.nblk_per_expert;
  const int nbk = blockIdx.x - e * p.nblk_per_expert;
  const int kp = nbk % p.kparts, nb = nbk / p.kparts;     // K part, column strip
  int row0 = 0, cnt = p.rows;
  if (p.offsets) {
    row0 = p.offsets[e];
    cnt = p.offsets[e + 1] - row0;
  }
  row0 = __builtin_amdgcn_readfirstlane(row0);
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  if (cnt <= 0) return;
  const int n0 = nb * NOUT;
  const int r16 = lane & 15, g = lane >> 4;
  const int KP = p.K / p.kparts, K0 = kp * KP;            // this block's K range
  const int iters = KP / KI;
  const int G = KP >> 7, GP = G + 1, g0 = K0 >> 7, Gall = p.K >> 7;
  const uint32_t row_bytes = INT4 ? (uint32_t)p.K / 2 : (uint32_t)p.K * 2;
  const uint32_t k0_bytes = INT4 ? (uint32_t)K0 / 2 : (uint32_t)K0 * 2;

  // weight strips: rows n0 .. n0+NOUT of each matrix (gate/up: gate and up)
  const uint32_t strip_bytes = (uint32_t)min(NOUT, p.N - n0) * row_bytes;
  const __amdgpu_buffer_rsrc_t wres0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.W0 + ((size_t)e * p.N + n0) * row_bytes), (short)0, (int)strip_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t wres1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((MODE == kSModeGateUp ? p.W1 : p.W0) + ((size_t)e * p.N + n0) * row_bytes), (short)0,
      (int)strip_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.X, (short)0, (int)p.xbytes, 0x00020000);
  // strip row of row block rb of wave w (gate/up: blocks RBW/2.. are the up rows
  // of the same f-values as blocks 0..)
  auto strip_row = [&](int ww, int rb) {
    return MODE == kSModeGateUp ? ww * NWF + (rb % (RBW / 2)) * 16 : ww * NWF + rb * 16;
  };
  auto second = [](int rb) { return MODE == kSModeGateUp && rb >= RBW / 2; };
  uint32_t wvoff[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
    wvoff[rb] = (uint32_t)(strip_row(w, rb) + r16) * row_bytes + k0_bytes + (uint32_t)g * 16;

  bool fused_ok = true;
  if constexpr (INT4) {
    // scale table row br = ww*RBW*16 + rb*16 + r: strip row strip_row(ww, rb) + r,
    // the G groups of this block's K range.  VG groups (2*VG bytes of scales,
    // as many of zero points) per load, all of a thread's loads issued
    // together: one memory round trip.  VG = 8 when p.sz_vec (G % 8 == 0 and
    // 16-byte aligned arrays), else 4 (the launcher checks G % 4 == 0, G <= 64
    // and 8-byte alignment)
    bool ok = true;
    auto stage = [&](auto vg) {
      constexpr int VG = decltype(vg)::value;
      typedef uint32_t vec_t __attribute__((ext_vector_type(VG / 2)));
      const int GV = G / VG;
      const int nload = 4 * RBW * 16 * GV;  // loads per array (uniform)
      constexpr int kMaxPer = RBW * 16 / VG;  // 64*RBW rows * (G <= 64)/VG loads over 256 threads
      vec_t sv[kMaxPer], zv[kMaxPer];
#pragma unroll
      for (int q = 0; q < kMaxPer; ++q) {
        if (q * 256 >= nload) break;
        const int i = tid + q * 256;
        sv[q] = zv[q] = vec_t{};
        if (i < nload) {
          const int br = i / GV, j = i - br * GV;
          const int ww = br / (RBW * 16), rb = (br / 16) % RBW, r = br % 16;
          const int n = n0 + strip_row(ww, rb) + r;
          if (n < p.N) {
            const size_t o = ((size_t)e * p.N + n) * Gall + g0 + j * VG;
            sv[q] = *(const vec_t*)((second(rb) ? p.s1 : p.s0) + o);
            zv[q] = *(const vec_t*)((second(rb) ? p.z1 : p.z0) + o);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kMaxPer; ++q) {
        if (q * 256 >= nload) break;
        const int i = tid + q * 256;
        if (i < nload) {
          const int br = i / GV, j = i - br * GV;
#pragma unroll
          for (int h = 0; h < VG / 2; ++h) {
            const uint32_t s2 = sv[q][h], z2 = zv[q][h];
            ok = ok && zero_point_fma_exact((u16)(z2 & 0xffffu)) && zero_point_fma_exact((u16)(z2 >> 16));
            sz[br * GP + j * VG + 2 * h] = (s2 & 0xffffu) | (z2 << 16);
            sz[br * GP + j * VG + 2 * h + 1] = (s2 >> 16) | (z2 & 0xffff0000u);
          }
        }
      }
    };
    if (p.sz_vec)
      stage(std::integral_constant<int, 8>{});
    else
      stage(std::integral_constant<int, 4>{});
    // the fused decode when every zero point of the block allows it (the usual
    // case), else the two-operation form; uniform over the block
    fused_ok = __syncthreads_and(ok) != 0;
  }

  auto body = [&](auto fused) {
    for (int mbase = 0; mbase < cnt; mbase += MB * 16) {
      const int mrows = min(MB * 16, cnt - mbase);
      // a pass of at most 16 rows runs its first 16-row token block only (MBE = 1):
      // no loads, LDS traffic or MFMAs for the clamped copies
      auto pass = [&](auto mbe_c) {
        constexpr int MBE = decltype(mbe_c)::value;
        // token slice loads: thread (q, c, tid) copies 16-byte chunk c*16 + tid%16
        // of token row q*16 + tid/16
        uint32_t xv[MBE];
#pragma unroll
        for (int q = 0; q < MBE; ++q) {
          const int rr = row0 + mbase + min(q * 16 + (tid >> 4), mrows - 1);  // clamped copies
          const int src = p.gather ? p.gather[rr] / p.k : rr;
          xv[q] = ((uint32_t)src * (uint32_t)p.ldx + (uint32_t)K0 + (uint32_t)(tid & 15) * 8) * 2u;
        }
        if constexpr (MODE == kSModeDown) {
          // gates of this pass's rows, published by the first slice's barrier
          if (tid < MB * 16) {
            const int rr = row0 + mbase + min(tid, mrows - 1);
            gsm[tid] = p.gate ? p.gate[p.gate_map ? p.gate_map[rr] : rr] : 1.0f;
          }
        }
        f32x4 acc[RBW][MBE];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
          for (int mb = 0; mb < MBE; ++mb) acc[rb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

        struct Set {
          u32x4 wv[RBW][WL];
        };
        auto load = [&](Set& S, int it) {
          const bool live = it < iters;  // uniform
          const uint32_t wo = live ? (uint32_t)it * IT_BYTES : strip_bytes;
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int q = 0; q < WL; ++q)
              S.wv[rb][q] = __builtin_bit_cast(
                  u32x4, __builtin_amdgcn_raw_buffer_load_b128(second(rb) ? wres1 : wres0,
                                                               (int)(wvoff[rb] + wo + q * 64), 0, 0));
          __builtin_amdgcn_sched_barrier(0);
        };
        // the token slice (from L2) is loaded one slice ahead, ahead of the
        // weight loads issued after it, so waiting for it never waits for them
        u32x4 xr[MBE][WQ];
        auto load_x = [&](int it) {
          const bool live = it < iters;  // uniform
#pragma unroll
          for (int q = 0; q < MBE; ++q)
#pragma unroll
            for (int c = 0; c < WQ; ++c)
              xr[q][c] = __builtin_bit_cast(
                  u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                             xres, (int)(live ? xv[q] + (uint32_t)it * KI * 2 + c * 256 : p.xbytes),
                             0, 0));
          __builtin_amdgcn_sched_barrier(0);
        };
        auto compute = [&](const Set& S, const unsigned char* slot, int it) {
          // sub-slice q = 128 K values (one INT4 group); token fragments: lane (t, g),
          // step s reads K q*128 + [g*32 + s*8, +8) (INT4) or [s*32 + g*8, +8) (bf16)
          // of token row t, as the weight lanes do
#pragma unroll
          for (int q = 0; q < WQ; ++q) {
            u32x4 xf[MBE][NS];
#pragma unroll
            for (int mb = 0; mb < MBE; ++mb)
#pragma unroll
              for (int s = 0; s < NS; ++s)
                xf[mb][s] = *(const u32x4*)(slot + (mb * 16 + r16) * XROW +
                                            (q * 128 + (INT4 ? g * 32 + s * 8 : s * 32 + g * 8)) * 2);
            if constexpr (!INT4) {
#pragma unroll
              for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                for (int s = 0; s < NS; ++s)
#pragma unroll
                  for (int mb = 0; mb < MBE; ++mb)
                    acc[rb][mb] = mfma16(as_bf16x8(S.wv[rb][s]), as_bf16x8(xf[mb][s]), acc[rb][mb]);
            } else {
              const int grp = min(it, iters - 1) * WQ + q;  // past the K range the tokens are zeros
#pragma unroll
              for (int rb = 0; rb < RBW; ++rb) {
                const uint32_t v = sz[(w * RBW * 16 + rb * 16 + r16) * GP + grp];
                const float sf = h2f((u16)(v & 0xffffu)), zf = h2f((u16)(v >> 16));
                const float nzs = -(zf * sf);
                bf16x8 a[NS];
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                  if constexpr (decltype(fused)::value)
                    a[s] = dq8_mix(S.wv[rb][q][s], sf, nzs);
                  else
                    a[s] = dq8_exact(S.wv[rb][q][s], sf, zf);
                }
#pragma unroll
                for (int s = 0; s < NS; ++s)
#pragma unroll
                  for (int mb = 0; mb < MBE; ++mb)
                    acc[rb][mb] = mfma16(a[s], as_bf16x8(xf[mb][s]), acc[rb][mb]);
              }
            }
            // one sub-slice's token fragments live at a time
            __builtin_amdgcn_sched_barrier(0);
          }
        };

        // slice it: weight register set it % D (loaded D slices ahead), LDS slot
        // it % 2.  Slot it % 2 was last read in slice it - 2, which every wave
        // finished before the barrier of slice it - 1.
        Set st[D];
        load_x(0);
#pragma unroll
        for (int d = 0; d < D; ++d) load(st[d], d);
        for (int it0 = 0; it0 < iters; it0 += D) {
#pragma unroll
          for (int u = 0; u < D; ++u) {
            const int it = it0 + u;
            unsigned char* slot = xs + (u & 1) * XSLOT;  // it0 is even when D is
            if (D % 2 != 0) slot = xs + (it & 1) * XSLOT;
#pragma unroll
            for (int q = 0; q < MBE; ++q)
#pragma unroll
              for (int c = 0; c < WQ; ++c)
                *(u32x4*)(slot + (q * 16 + (tid >> 4)) * XROW + (c * 16 + (tid & 15)) * 16) = xr[q][c];
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
            block_barrier();
            load_x(it + 1);
            compute(st[u], slot, it);
            load(st[u], it + D);
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // epilogue from the accumulators: lane (t, g) holds weight rows 4g..4g+3
        // of each row block for token row t (C layout of the 16x16 MFMA)
#pragma unroll
        for (int mb = 0; mb < MBE; ++mb) {
          const int row = mbase + mb * 16 + r16;
          if (row >= cnt) continue;
          const size_t orow = (size_t)(row0 + row);
          constexpr int NOB = (MODE == kSModeGateUp) ? RBW / 2 : RBW;
#pragma unroll
          for (int ob = 0; ob < NOB; ++ob) {
            const int f = n0 + w * NWF + ob * 16 + 4 * g;
            if (f >= p.N) continue;
            if constexpr (MODE == kSModeDown) {
              const float gv = gsm[mb * 16 + r16];
              const f32x4 a = acc[ob][mb];
              *(f32x4*)(p.Y + (size_t)kp * p.ystride + orow * p.N + f) =
                  f32x4{gv * a[0], gv * a[1], gv * a[2], gv * a[3]};
              continue;
            }
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (MODE == kSModeGateUp)
                o[i] = silu_f32(acc[ob][mb][i]) * acc[ob + RBW / 2][mb][i];
              else
                o[i] = fmaxf(acc[ob][mb][i], 0.0f);
            }
            *(uint2*)(p.H + orow * p.N + f) = uint2{pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3])};
          }
        }
      };
      if (MB > 1 && mrows <= 16)
        pass(std::integral_constant<int, 1>{});
      else
        pass(std::integral_constant<int, MB>{});
      // the next pass writes slot 0 and the gates again
      if (mbase + MB * 16 < cnt) __syncthreads();
    }
  };
  if constexpr (INT4) {
    if (fused_ok)
      body(std::true_type{});
    else
      body(std::false_type{});
  } else {
    body(std::true_type{});
  }
}

// K: the K range of one block (K / parts)
template <int MODE, bool INT4, int MB, int WQ, int RBW = kRowsRBW>
size_t stream_rows_lds_bytes(int K) {
  return (size_t)2 * MB * 16 * rows_xrow(WQ) +
         (INT4 ? (size_t)4 * RBW * 16 * ((K >> 7) + 1) * 4 : 0);
}

template <int MODE, bool INT4>
size_t stream_reg_lds_bytes(int K) {
  constexpr int R = stream_reg_rows(MODE, INT4);
  return (size_t)4 * (R / 16) * 64 * 16 + (INT4 ? (size_t)R * ((K >> 7) + 1) * 4 : 0);
}

template <int MODE, bool INT4>
hipError_t launch_reg_mode(const StreamArgs& a0, int E, int mb, hipStream_t s) {
  constexpr int NOUT = MODE == kSModeGateUp ? stream_reg_rows(MODE, INT4) / 2 : stream_reg_rows(MODE, INT4);
  StreamArgs a = a0;
  a.nblk_per_expert = (a.N + NOUT - 1) / NOUT;
  a.sz_vec = 0;
  if constexpr (INT4) {
    constexpr int R = stream_reg_rows(MODE, INT4);
    auto al16 = [](const void* q) { return q == nullptr || ((uintptr_t)q % 16) == 0; };
    a.sz_vec = (a.K % 1024 == 0) && ((long long)R * (a.K / 1024) <= 2048) && al16(a.s0) &&
               al16(a.z0) && (MODE != kSModeGateUp || (al16(a.s1) && al16(a.z1)));
  }
  const dim3 grid((unsigned)(E * a.nblk_per_expert)), block(256);
  const size_t lds = stream_reg_lds_bytes<MODE, INT4>(a.K);
  // two register sets in flight: deeper prefetch measured no faster here
  if (mb <= 1)
    hipLaunchKernelGGL((stream_reg_kernel<MODE, INT4, 1, 2>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((stream_reg_kernel<MODE, INT4, 2, 2>), grid, block, lds, s, a);
  return hipGetLastError();
}

constexpr int kRowsWQ = 1;                 // INT4: K groups per slice (measured: 2 is slower)
constexpr int kRowsRBWUp = 2;              // 16-row weight blocks per wave: gate/up, ReLU W_in (2: measured ~5% faster than 4)
constexpr int kRowsRBWDown = 2;            // and down (2 with 4 K parts: ~5% faster than 4)
constexpr size_t kRowsMaxLds = 80 * 1024;  // two blocks per CU

template <int MODE, bool INT4, int RBW>
hipError_t launch_rows_mode(const StreamArgs& a0, int E, int mb, int parts, hipStream_t s) {
  constexpr int NOUT = stream_rows_nout<MODE, RBW>();
  constexpr int WQ = INT4 ? kRowsWQ : 1;
  StreamArgs a = a0;
  a.kparts = parts;
  a.nblk_per_expert = (a.N + NOUT - 1) / NOUT * parts;
  auto al16 = [](const void* q) { return q == nullptr || ((uintptr_t)q % 16) == 0; };
  a.sz_vec = INT4 && ((a.K / parts) >> 7) % 8 == 0 && al16(a.s0) && al16(a.z0) && al16(a.s1) &&
             al16(a.z1);
  const dim3 grid((unsigned)(E * a.nblk_per_expert)), block(256);
  auto k1 = stream_rows_kernel<MODE, INT4, 1, 2, WQ, RBW>;
  auto k2 = stream_rows_kernel<MODE, INT4, 2, 2, WQ, RBW>;
  // the dynamic-LDS limit of both instantiations is raised once per device,
  // under a lock, so concurrent first calls from several threads are safe
  static std::mutex attr_mu;
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lk(attr_mu);
    const bool cached = dev >= 0 && dev < 64;
    if (!cached || !attr_set[dev]) {
      e = hipFuncSetAttribute((const void*)k1, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kRowsMaxLds);
      if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)k2, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)kRowsMaxLds);
      if (e != hipSuccess) return e;
      if (cached) attr_set[dev] = true;
    }
  }
  const size_t lds1 = stream_rows_lds_bytes<MODE, INT4, 1, WQ, RBW>(a.K / parts);
  const size_t lds2 = stream_rows_lds_bytes<MODE, INT4, 2, WQ, RBW>(a.K / parts);
  if (mb <= 1)
    hipLaunchKernelGGL(k1, grid, block, lds1, s, a);
  else
    hipLaunchKernelGGL(k2, grid, block, lds2, s, a);
  return hipGetLastError();
}

template <int MODE, bool INT4>
hipError_t launch_mode(const StreamArgs& a, int E, int mb, hipStream_t s) {
  const dim3 grid((unsigned)(E * a.nblk_per_expert)), block(256);
  // up to 32 token rows per pass; an expert with more rows takes further passes
  if (mb <= 1)
    hipLaunchKernelGGL((stream_ffn_kernel<MODE, INT4, 1>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((stream_ffn_kernel<MODE, INT4, 2>), grid, block, 0, s, a);
  return hipGetLastError();
}

// ---- INT4 -> bf16 decode of whole projections ---------------------------------
// The many-row replica slot runs the bf16 tile kernels on a decoded copy of its
// INT4 weights: one thread decodes one word (8 weights) with the same rule as
// the GEMM kernels (fused form when the group's zero point allows it, else the
// two-operation form) and writes 16 bytes.
__global__ __launch_bounds__(256) void dequant_int4_kernel(const uint32_t* __restrict__ q,
                                                           const u16* __restrict__ s,
                                                           const u16* __restrict__ z, size_t words,
                                                           int K, u16* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= words) return;
  const size_t kw = (size_t)K / 8;
  const size_t row = i / kw, kk = (i - row * kw) * 8;
  const size_t gi = row * (size_t)(K >> 7) + (kk >> 7);
  const u16 zh = z[gi];
  const float sf = h2f(s[gi]), zf = h2f(zh);
  const uint32_t w = q[i];
  const bf16x8 v = zero_point_fma_exact(zh) ? dq8_mix(w, sf, -(zf * sf)) : dq8_exact(w, sf, zf);
  *(bf16x8*)(out + i * 8) = v;
}

}  // namespace

// The row-split INT4 kernel over K range K / parts: its token slices and scale
// table fit the LDS limit, the table stages with 8-byte loads (4 groups: the
// range is a multiple of 512), scales and zero points 8-byte aligned
bool stream_rows_applies(int K, int parts, const moe_w4* a, const moe_w4* b) {
  if (parts < 1 || K % parts != 0) return false;
  const int KP = K / parts;
  auto al8 = [](const void* q) { return q != nullptr && ((uintptr_t)q % 8) == 0; };
  return KP % 512 == 0 && KP <= 8192 &&
         stream_rows_lds_bytes<kSModeGateUp, true, 2, kRowsWQ>(KP) <= kRowsMaxLds && a && b &&
         al8(a->scale) && al8(a->zero) && al8(b->scale) && al8(b->zero);
}

int stream_down_parts(int d, int F, int E) {
  // about four blocks per CU: E * ceil(d / strip rows) strips times the parts
  constexpr int NOUT = stream_rows_nout<kSModeDown, kRowsRBWDown>();
  const long long strips = (long long)E * ((d + NOUT - 1) / NOUT);
  for (int P = 8; P > 1; P /= 2)
    if (F % (512 * P) == 0 && strips * P <= 4 * 256 && F / P <= 8192) return P;
  return 1;
}

hipError_t launch_dequant_int4(const moe_w4* w, int rows, int K, void* out, hipStream_t s) {
  if (K % 128 != 0) return hipErrorInvalidValue;
  const size_t words = (size_t)rows * (K / 8);
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_int4_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                     (const uint32_t*)w->q, w->scale, w->zero, words, K, (u16*)out);
  return hipGetLastError();
}

bool stream_ffn_applies(const FfnProblem& p) {
  if (p.dt != MOE_DT_BF16) return false;
  // few rows per expert: every expert has at most T rows (a token picks an
  // expert once); beyond 64 the tiled kernels win
  if (p.T > 64) return false;
  // chunking needs both reduction lengths to be multiples of 512
  return (p.d % 512) == 0 && (p.F % 512) == 0;
}

hipError_t launch_stream_ffn(const FfnProblem& p, hipStream_t s, hipEvent_t mid) {
  const bool int4 = p.w->q_up != nullptr;
  const bool relu = p.act == MOE_ACT_RELU;
  const int E = p.offsets ? p.E : 1;
  const int mb = (p.T + 15) / 16;
  StreamArgs a{};
  a.k = p.k;
  a.offsets = p.offsets;
  a.rows = p.rows;
  // gate/up (or ReLU W_in): weights [E][F][d], tokens x
  a.X = (const u16*)p.x;
  a.ldx = p.d;
  a.gather = p.row_assign;
  a.N = p.F;
  a.K = p.d;
  a.H = (u16*)p.H;
  a.zero = (f32x4*)p.zero_y;
  a.zero_n4 = p.zero_y ? (size_t)p.T * p.d / 4 : 0;
  a.nblk_per_expert = (p.F + 31) / 32;
  // the register-direct kernel addresses the token matrix (x, then H) and a
  // weight strip of up to 64 rows with 32-bit buffer offsets
  const size_t xb = (size_t)p.T * p.d * 2, hb = (size_t)p.rows * p.F * 2;
  const size_t strip = 64 * (size_t)(p.d > p.F ? p.d : p.F) * (int4 ? 1 : 4) / 2;
  const bool reg = xb < (1u << 31) && hb < (1u << 31) && strip < (1u << 31);
  // INT4 gate/up and ReLU W_in: the row-split kernel (see stream_rows_applies)
  const bool rows = reg && int4 &&
                    stream_rows_applies(p.d, 1, relu ? p.w->q_up : p.w->q_gate, p.w->q_up);
  a.xbytes = (uint32_t)xb;
  if (int4) {
    const moe_w4* g = relu ? p.w->q_up : p.w->q_gate;
    const moe_w4* u = p.w->q_up;
    a.W0 = (const unsigned char*)g->q; a.s0 = g->scale; a.z0 = g->zero;
    a.W1 = (const unsigned char*)u->q; a.s1 = u->scale; a.z1 = u->zero;
  } else {
    a.W0 = (const unsigned char*)(relu ? p.w->w_up : p.w->w_gate);
    a.W1 = (const unsigned char*)p.w->w_up;
  }
  hipError_t e;
  if (relu)
    e = int4 ? (rows  ? launch_rows_mode<kSModeRelu, true, kRowsRBWUp>(a, E, mb, 1, s)
                : reg ? launch_reg_mode<kSModeRelu, true>(a, E, mb, s)
                      : launch_mode<kSModeRelu, true>(a, E, mb, s))
             : (reg ? launch_reg_mode<kSModeRelu, false>(a, E, mb, s)
                    : launch_mode<kSModeRelu, false>(a, E, mb, s));
  else
    e = int4 ? (rows  ? launch_rows_mode<kSModeGateUp, true, kRowsRBWUp>(a, E, mb, 1, s)
                : reg ? launch_reg_mode<kSModeGateUp, true>(a, E, mb, s)
                      : launch_mode<kSModeGateUp, true>(a, E, mb, s))
             : (reg ? launch_reg_mode<kSModeGateUp, false>(a, E, mb, s)
                    : launch_mode<kSModeGateUp, false>(a, E, mb, s));
  if (e != hipSuccess) return e;
  if (mid) {
    e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
  }
  // down: weights [E][d][F], operand H
  StreamArgs b{};
  b.k = p.k;
  b.offsets = p.offsets;
  b.rows = p.rows;
  b.X = (const u16*)p.H;
  b.ldx = p.F;
  b.gather = nullptr;
  b.N = p.d;
  b.K = p.F;
  b.Y = p.y_rows;
  b.Yacc = p.y_direct;
  b.xbytes = (uint32_t)hb;
  b.gate_map = p.row_assign;
  b.gate = p.gate;
  b.nblk_per_expert = (p.d + 31) / 32;
  if (int4) {
    b.W0 = (const unsigned char*)p.w->q_down->q; b.s0 = p.w->q_down->scale; b.z0 = p.w->q_down->zero;
  } else {
    b.W0 = (const unsigned char*)p.w->w_down;
  }
  // bf16 down rows are long (K = d_ff): whole contiguous row pieces staged
  // through LDS stream faster there than MFMA-shaped register loads
  if (int4 && reg && p.down_splits > 1) {
    // K split into parts: partial rows to y_rows + part * rows * d, which the
    // combine adds (the layer sized y_rows and chose the parts for this)
    if (!stream_rows_applies(p.F, p.down_splits, p.w->q_down, p.w->q_down))
      return hipErrorInvalidValue;
    b.ystride = (size_t)p.rows * p.d;
    return launch_rows_mode<kSModeDown, true, kRowsRBWDown>(b, E, mb, p.down_splits, s);
  }
  if (int4 && reg) return launch_reg_mode<kSModeDown, true>(b, E, mb, s);
  return int4 ? launch_mode<kSModeDown, true>(b, E, mb, s) : launch_mode<kSModeDown, false>(b, E, mb, s);
}

}  // namespace moe
