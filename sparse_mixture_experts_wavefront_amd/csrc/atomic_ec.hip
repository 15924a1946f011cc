// atomic_ec.hip -- expert-centric execution of atomic experts.
//
// "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale" -- What
// carries the argument and Figure 3: execution is inverted from token order to
// expert order; the kept (token, expert) pairs are grouped by expert (offsets,
// rows in token order), so each expert's parameters are read once and applied
// to all of its tokens, instead of every token fetching its scattered experts.
// An atomic expert n is one vector pair: for a kept pair (t, n) with gate g,
// h = bf16_RNE(g * silu(x[t] . w_in[n])) and the token receives h * w_out[n].
//
// Input side (one wave per expert with rows): the wave loads w_in[n] once into
// registers (d/64 values per lane) and walks the expert's rows; each row is
// one dot product with x[t] (bf16 pairs into fp32 with v_dot2, then a sum over
// the 64 lanes).  h is written in row order.
// Output side: a block owns a range of experts, a chunk of 16 tokens and a
// slice of output columns.  It lists the experts of its range that have rows
// in its token chunk, streams each listed expert's output vector once (from
// the unit-major copy w_out_rows [N][d], 16 bytes per lane, D experts ahead)
// and adds h * w_out[n] into per-token fp32 accumulators in LDS (each thread
// its own 8 columns of every token).  Each range leaves partial sums of its
// experts; the reduce kernel adds the ranges in range order, then the shared
// MLP's rows, so the result is run-to-run deterministic.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kEcInUnits = 32;         // consecutive experts per block (input side)
constexpr int kEcInRows = 512;         // their rows staged in LDS (32 experts x 16 tokens)
constexpr int kEcOutThreads = 64;       // output side: threads per block (one wave)
constexpr int kEcOutCols = 8;           // columns per thread (one 16-byte bf16 load)
constexpr int kEcOutSlice = kEcOutThreads * kEcOutCols;   // 512 columns per block
constexpr int kEcTok = 16;              // tokens per output-side block
constexpr int kEcList = 256;            // experts listed per round of the output side
constexpr int kEcAhead = 32;            // output vectors in flight per thread
constexpr int kEcOutRows = 512;         // rows of a listing round staged in LDS (T <= 16)

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a),
                                         __builtin_bit_cast(bf16x2v, b), c, false);
}
// the four words by name: a loop over a[q] here let the compiler use word 0 four
// times (seen in the generated code), so each element is spelled out
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float c) {
  c = dot2(a.x, b.x, c);
  c = dot2(a.y, b.y, c);
  c = dot2(a.z, b.z, c);
  return dot2(a.w, b.w, c);
}

// sum over the 64 lanes, the same value in every lane: DPP adds inside each
// row of 16 lanes (swap neighbours, swap pairs, mirror halves of 8, mirror the
// row), then the four row sums read out and added in row order
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xb1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4e>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

// NC = d / 512: a lane holds K values [c*512 + lane*8, +8) of chunk c.
// Block = kEcInUnits consecutive experts; their rows are one contiguous range
// of the grouping.  When that range fits the LDS (always for T <= 16), the
// rows' tokens and gates are staged there first in one coalesced pass, so a
// wave's work per expert is its w_in load (issued one expert ahead) and the x
// rows (L2), with no dependent loads of the grouping in the way.
template <int NC>
__global__ __launch_bounds__(256) void atomic_ec_in_kernel(
    const u16* __restrict__ x, const u16* __restrict__ w_in, int N,
    const int32_t* __restrict__ off, const int32_t* __restrict__ row_assign,
    const float* __restrict__ gates, int K, u16* __restrict__ h) {
  constexpr int d = 512 * NC;
  __shared__ int s_off[kEcInUnits + 1];
  __shared__ int s_tok[kEcInRows];
  __shared__ float s_gate[kEcInRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u0 = blockIdx.x * kEcInUnits;
  const int nu = min(kEcInUnits, N - u0);
  for (int i = tid; i <= nu; i += 256) s_off[i] = off[u0 + i];
  __syncthreads();
  const int rbase = s_off[0], nrows = s_off[nu] - rbase;
  const bool staged = nrows <= kEcInRows;  // uniform
  if (staged) {
    for (int i = tid; i < nrows; i += 256) {
      const int a = row_assign[rbase + i];
      s_tok[i] = a / K;
      s_gate[i] = gates[a];
    }
  }
  __syncthreads();

  auto next_active = [&](int i) {
    while (i < nu && s_off[i] == s_off[i + 1]) i += 4;
    return i;
  };
  auto load_w = [&](u32x4 (&wv)[NC], int i) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
      wv[c] = *(const u32x4*)(w_in + (size_t)(u0 + i) * d + c * 512 + lane * 8);
  };
  struct Rows {
    int nr;
    float gt[4];
    u32x4 xv[4][NC];
  };
  // rows r .. r+3 (clamped to r1): tokens and gates, then their x loads
  auto gather = [&](Rows& g, int r, int r1, auto staged_tag) __attribute__((always_inline)) {
    g.nr = min(4, r1 - r);
    int tok[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = r + min(q, g.nr - 1);
      if constexpr (decltype(staged_tag)::value) {
        tok[q] = s_tok[rr - rbase];
        g.gt[q] = s_gate[rr - rbase];
      } else {
        const int a = __builtin_amdgcn_readfirstlane(row_assign[rr]);
        tok[q] = a / K;
        g.gt[q] = gates[a];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u16* xr = x + (size_t)tok[q] * d + lane * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) g.xv[q][c] = *(const u32x4*)(xr + c * 512);
    }
  };
  auto finish = [&](const Rows& g, int r, const u32x4 (&wv)[NC]) __attribute__((always_inline)) {
    float part[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float sum = 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c) sum = dot8(g.xv[q][c], wv[c], sum);
      part[q] = wave_sum(sum);
    }
    if (lane < g.nr) {
      const float u = lane == 0 ? part[0] : lane == 1 ? part[1] : lane == 2 ? part[2] : part[3];
      const float gg = lane == 0 ? g.gt[0] : lane == 1 ? g.gt[1] : lane == 2 ? g.gt[2] : g.gt[3];
      h[r + lane] = f32_to_bf16(gg * silu_f32(u));
    }
  };
  // expert i with w_in in wcur: the first rows' x loads go out before the
  // next expert's w_in (into wnxt), so the wait for them leaves that prefetch
  // in flight under this expert's work; returns the next expert
  auto one = [&](int i, const u32x4 (&wcur)[NC], u32x4 (&wnxt)[NC], auto staged_tag)
      __attribute__((always_inline)) {
    const int inext = next_active(i + 4);
    const int r0 = s_off[i], r1 = s_off[i + 1];
    Rows g;
    gather(g, r0, r1, staged_tag);
    load_w(wnxt, min(inext, nu - 1));  // unconditional: the waits stay counted
    finish(g, r0, wcur);
    for (int r = r0 + 4; r < r1; r += 4) {
      gather(g, r, r1, staged_tag);
      finish(g, r, wcur);
    }
    return inext;
  };
  // two register sets used in turn (a copy from one to the other would wait
  // for the prefetch right away)
  auto run = [&](auto staged_tag) __attribute__((always_inline)) {
    int i = next_active(w);
    u32x4 wa[NC], wb[NC];
    if (i < nu) load_w(wa, i);
    while (i < nu) {
      i = one(i, wa, wb, staged_tag);
      if (i >= nu) break;
      i = one(i, wb, wa, staged_tag);
    }
  };
  if (staged)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// first row of [r0, r1) (rows of one expert, tokens ascending) whose token is >= t
__device__ __forceinline__ int first_row_at(const int32_t* __restrict__ row_assign, int r0, int r1,
                                            int K, int t) {
  int lo = r0, hi = r1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row_assign[mid] / K < t) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// block = (expert range p, token chunk tc, column slice cs); grid-linear index
// ((p * ntc) + tc) * ncs + cs.  upr experts per range.  The per-token sums of a
// thread's 8 columns live in LDS (acc[token][column], each thread touching only
// its own columns, so no barrier guards them): a row of token t is two 16-byte
// LDS reads, eight FMAs and two writes at row t.
__global__ __launch_bounds__(kEcOutThreads) void atomic_ec_out_kernel(
    const u16* __restrict__ h, const int32_t* __restrict__ off,
    const int32_t* __restrict__ row_assign, int K, const u16* __restrict__ w_out_rows, int N,
    int d, int T, int upr, int ntc, int ncs, float* __restrict__ ypart) {
  __shared__ int lst_n[kEcList + kEcAhead], lst_r0[kEcList + kEcAhead], lst_r1[kEcList + kEcAhead];
  __shared__ int s_tl[kEcOutRows];    // staged rows of the round: token - t0
  __shared__ float s_h[kEcOutRows];   // and h
  __shared__ __align__(16) float acc[kEcTok][kEcOutSlice];
  const int tid = threadIdx.x, lane = tid;
  const int cs = blockIdx.x % ncs;
  const int rest = blockIdx.x / ncs;
  const int tc = rest % ntc, p = rest / ntc;
  const int u0 = p * upr, u1 = min(N, u0 + upr);
  const int t0 = tc * kEcTok;
  const int tn = min(kEcTok, T - t0);
  const int c8 = tid * kEcOutCols;              // this thread's columns in the slice
  const int col = cs * kEcOutSlice + c8;
  const bool colok = col < d;  // d % 8 == 0: a thread's 8 columns are all in or all out
  const bool narrow = T > kEcTok;

#pragma unroll
  for (int i = 0; i < kEcTok; ++i) {
    *(f32x4*)&acc[i][c8] = f32x4{0.f, 0.f, 0.f, 0.f};
    *(f32x4*)&acc[i][c8 + 4] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int base = u0; base < u1; base += kEcList) {
    // list the experts of this round that have rows in the token chunk (one
    // wave: a ballot gives each active lane its position)
    int cnt = 0;
    for (int q = 0; q < kEcList; q += kEcOutThreads) {
      const int n = base + q + tid;
      int r0 = 0, r1 = 0;
      if (n < u1) {
        r0 = off[n];
        r1 = off[n + 1];
        if (narrow && r0 < r1) {
          r0 = first_row_at(row_assign, r0, r1, K, t0);
          r1 = first_row_at(row_assign, r0, r1, K, t0 + kEcTok);
        }
      }
      const bool act = r0 < r1;
      const unsigned long long m = __ballot(act);
      if (act) {
        const int pos = cnt + __popcll(m & ((1ull << lane) - 1ull));
        lst_n[pos] = n;
        lst_r0[pos] = r0;
        lst_r1[pos] = r1;
      }
      cnt += __popcll(m);
    }
    if (cnt == 0) continue;  // uniform: no expert of this round has rows here
    // pad the list to a multiple of kEcAhead with row-less copies of its last
    // expert, so the streaming loop below issues every load unconditionally
    // (the compiler can then wait for the oldest load only)
    const int cntpad = (cnt + kEcAhead - 1) / kEcAhead * kEcAhead;
    __syncthreads();
    if (tid < cntpad - cnt) {
      lst_n[cnt + tid] = lst_n[cnt - 1];
      lst_r0[cnt + tid] = 0;
      lst_r1[cnt + tid] = 0;
    }
    // T <= 16: the round's rows are one contiguous range of the grouping;
    // stage their tokens and h in LDS in one coalesced pass
    int rb0 = 0;
    bool staged = false;
    if (!narrow) {
      rb0 = off[base];
      const int nrows = off[min(u1, base + kEcList)] - rb0;
      staged = nrows <= kEcOutRows;
      if (staged) {
        for (int j = tid; j < nrows; j += kEcOutThreads) {
          s_tl[j] = row_assign[rb0 + j] / K;
          s_h[j] = bf16_to_f32(h[rb0 + j]);
        }
      }
    }
    __syncthreads();  // the padded list and the staged rows are visible
    // stream the listed experts' output vectors, kEcAhead in flight; the
    // staged variant has no other global loads in its loop, so the waits for
    // an output vector leave the younger ones in flight
    auto stream = [&](auto staged_tag) __attribute__((always_inline)) {
      constexpr bool STAGED = decltype(staged_tag)::value;
      u32x4 wq[kEcAhead];
      const u16* wbase = w_out_rows + (colok ? col : 0);
      // issued in list order (the scheduler must not reorder them: the loop
      // waits for the oldest one only)
#pragma unroll
      for (int i = 0; i < kEcAhead; ++i) {
        wq[i] = *(const u32x4*)(wbase + (size_t)lst_n[i] * d);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int m0 = 0; m0 < cntpad; m0 += kEcAhead) {
#pragma unroll
        for (int i = 0; i < kEcAhead; ++i) {
          const int m = m0 + i;
          const u32x4 wcur = wq[i];
          // the vector kEcAhead places on (the last one again past the list)
          wq[i] = *(const u32x4*)(wbase + (size_t)lst_n[min(m + kEcAhead, cntpad - 1)] * d);
          __builtin_amdgcn_sched_barrier(0);
          const int r1 = lst_r1[m];
          for (int r = lst_r0[m]; r < r1; ++r) {
            int tl;
            float hv;
            if constexpr (STAGED) {
              tl = s_tl[r - rb0];
              hv = s_h[r - rb0];
            } else {
              const int a = row_assign[r];
              tl = a / K - t0;
              hv = bf16_to_f32(h[r]);
            }
            float* ap = &acc[tl][c8];
            f32x4 lo = *(f32x4*)ap, hi = *(f32x4*)(ap + 4);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              lo[2 * q] = __builtin_fmaf(hv, __uint_as_float(wcur[q] << 16), lo[2 * q]);
              lo[2 * q + 1] = __builtin_fmaf(hv, __uint_as_float(wcur[q] & 0xffff0000u), lo[2 * q + 1]);
              hi[2 * q] = __builtin_fmaf(hv, __uint_as_float(wcur[q + 2] << 16), hi[2 * q]);
              hi[2 * q + 1] =
                  __builtin_fmaf(hv, __uint_as_float(wcur[q + 2] & 0xffff0000u), hi[2 * q + 1]);
            }
            *(f32x4*)ap = lo;
            *(f32x4*)(ap + 4) = hi;
          }
        }
      }
    };
    if (staged)
      stream(std::true_type{});
    else
      stream(std::false_type{});
    __syncthreads();  // the list is rebuilt next round
  }
  if (!colok) return;
  for (int i = 0; i < tn; ++i) {
    float* o = ypart + ((size_t)p * T + t0 + i) * d + col;
    *(f32x4*)o = *(const f32x4*)&acc[i][c8];
    *(f32x4*)(o + 4) = *(const f32x4*)&acc[i][c8 + 4];
  }
}

// y[t][cols] = sum over ranges p = 0..P-1 (in that order) of ypart[p][t][cols],
// then + y_shared[t][cols].  Block = (token, 256 columns); wave w adds the ranges
// [w*P/16, (w+1)*P/16) in order, the 16 wave sums are added in wave order.
template <bool BF16OUT>
__global__ __launch_bounds__(1024) void atomic_ec_reduce_kernel(const float* __restrict__ ypart,
                                                                int P, int T, int d,
                                                                const float* __restrict__ y_shared,
                                                                void* __restrict__ yv) {
  __shared__ f32x4 part[16][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nchunk = (d + 255) / 256;
  const int t = blockIdx.x / nchunk;
  const int i = (blockIdx.x % nchunk) * 256 + lane * 4;
  const bool ok = i < d;
  const int p0 = (int)((long long)w * P / 16), p1 = (int)((long long)(w + 1) * P / 16);
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ok) {
    int p = p0;
    for (; p + 4 <= p1; p += 4) {
      f32x4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *(const f32x4*)(ypart + ((size_t)(p + q) * T + t) * d + i);
#pragma unroll
      for (int q = 0; q < 4; ++q) s += v[q];
    }
    for (; p < p1; ++p) s += *(const f32x4*)(ypart + ((size_t)p * T + t) * d + i);
  }
  part[w][lane] = s;
  __syncthreads();
  if (w != 0 || !ok) return;
  f32x4 y = part[0][lane];
#pragma unroll
  for (int q = 1; q < 16; ++q) y += part[q][lane];
  if (y_shared) y += *(const f32x4*)(y_shared + (size_t)t * d + i);
  if constexpr (BF16OUT) {
    u16* o = (u16*)yv + (size_t)t * d + i;
    *(uint2*)o = make_uint2(pk_bf16(y[0], y[1]), pk_bf16(y[2], y[3]));
  } else {
    *(f32x4*)((float*)yv + (size_t)t * d + i) = y;
  }
}

}  // namespace

bool atomic_ec_supported(int d) { return d % 512 == 0 && d >= 512 && d <= 4096; }

int atomic_ec_ranges(int T, int d, int N) {
  // experts per range: at most kEcList per listing round; the partial sums
  // (ranges x T x d fp32) are capped near 256 MiB by using fewer, longer ranges
  const long long per = (long long)T * d * 4;
  long long P = (N + kEcList - 1) / kEcList;
  const long long cap = per > 0 ? ((256ll << 20) / per) : P;
  if (P > cap) P = cap < 1 ? 1 : cap;
  return (int)P;
}

size_t atomic_ec_ws_bytes(int T, int d, int N, int K) {
  const size_t hbytes = ((size_t)T * K * 2 + 255) & ~(size_t)255;
  return hbytes + (size_t)atomic_ec_ranges(T, d, N) * T * d * 4;
}

hipError_t launch_atomic_ec_in(const u16* x, int T, int d, const u16* w_in, int N,
                               const int32_t* offsets, const int32_t* row_assign,
                               const float* gates, int K, u16* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((N + kEcInUnits - 1) / kEcInUnits)), block(256);
  switch (d / 512) {
    case 1: hipLaunchKernelGGL(atomic_ec_in_kernel<1>, grid, block, 0, s, x, w_in, N, offsets, row_assign, gates, K, h); break;
    case 2: hipLaunchKernelGGL(atomic_ec_in_kernel<2>, grid, block, 0, s, x, w_in, N, offsets, row_assign, gates, K, h); break;
    case 4: hipLaunchKernelGGL(atomic_ec_in_kernel<4>, grid, block, 0, s, x, w_in, N, offsets, row_assign, gates, K, h); break;
    case 8: hipLaunchKernelGGL(atomic_ec_in_kernel<8>, grid, block, 0, s, x, w_in, N, offsets, row_assign, gates, K, h); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_atomic_ec_out(const u16* h, const int32_t* offsets, const int32_t* row_assign,
                                int K, const u16* w_out_rows, int N, int d, int T, float* ypart,
                                hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int P = atomic_ec_ranges(T, d, N);
  const int upr = (N + P - 1) / P;
  const int ntc = (T + kEcTok - 1) / kEcTok;
  const int ncs = (d + kEcOutSlice - 1) / kEcOutSlice;
  const long long blocks = (long long)P * ntc * ncs;
  if (blocks >= (1ll << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(atomic_ec_out_kernel, dim3((unsigned)blocks), dim3(kEcOutThreads), 0, s, h,
                     offsets, row_assign, K, w_out_rows, N, d, T, upr, ntc, ncs, ypart);
  return hipGetLastError();
}

hipError_t launch_atomic_ec_reduce(const float* ypart, int T, int d, int N,
                                   const float* y_shared, void* y, moe_dtype ydt, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int P = atomic_ec_ranges(T, d, N);
  const long long rb = (long long)T * ((d + 255) / 256);
  if (rb >= (1ll << 31)) return hipErrorInvalidValue;
  if (ydt == MOE_DT_BF16)
    hipLaunchKernelGGL(atomic_ec_reduce_kernel<true>, dim3((unsigned)rb), dim3(1024), 0, s, ypart,
                       P, T, d, y_shared, y);
  else
    hipLaunchKernelGGL(atomic_ec_reduce_kernel<false>, dim3((unsigned)rb), dim3(1024), 0, s,
                       ypart, P, T, d, y_shared, y);
  return hipGetLastError();
}

}  // namespace moe
