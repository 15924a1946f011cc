// route_topk.hip -- router logits and exact top-k with softmax gates.
//
// "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale" -- Core
// claim (each token scores every expert and keeps its top-K units) and Axiom
// ledger (the selection is the exact top-K, not an approximation).  Gates are the
// softmax over the k selected logits so each token's weights sum to one.
//
// One workgroup owns 16 tokens.  The logits of those tokens are a 16 x E tile of
// x . W_r^T.  For bf16 layers the NW waves of the group split the reduction
// over d (wave w takes the 32-wide K steps w, w+NW, ...), each with 16x16x32
// MFMA (fp32 accumulate), and the partial tiles meet in LDS in a fixed wave
// order; fp32 layers use fp32 FMA.  Many waves per token group keep a small
// batch (decode) from being one serial walk over d.  Selection then runs with
// one lane per expert: a wave is split into segments of SEG = next_pow2(E)
// lanes, one token per segment, and each of the k rounds is a butterfly max
// over a 64-bit key (order-preserving bits of the fp32 logit << 32 | (SEG-1-e)),
// so the largest logit wins and equal logits go to the lower expert id.  -0.0 is
// folded into +0.0 before keying, so the two compare equal.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokPerWave = 16;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_inv(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  uint32_t lo = __shfl_xor((int)(uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// EB: expert blocks of 16 columns covered by the MFMA logits tile (E <= 16*EB);
// NW: waves per workgroup.
template <int EB, int NW, bool F32>
__global__ __launch_bounds__(64 * NW) void route_topk_kernel(const void* __restrict__ xv,
                                                             const void* __restrict__ wv,
                                                             const float* __restrict__ bias, int T,
                                                             int d, int E, int k, int seg,
                                                             float* __restrict__ logits,
                                                             int32_t* __restrict__ idx,
                                                             float* __restrict__ gate,
                                                             int logits_given) {
  __shared__ float lt[kTokPerWave][kMaxExperts + 1];
  __shared__ f32x4 part[F32 ? 1 : NW][EB][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * kTokPerWave;

  if (!logits_given) {
    if constexpr (!F32) {
      const u16* x = (const u16*)xv;
      const u16* w = (const u16*)wv;
      const int r = lane & 15, g = lane >> 4;
      const int tok = min(t0 + r, T - 1);
      const u16* xr = x + (size_t)tok * d + g * 8;
      const u16* wr[EB];
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) wr[eb] = w + (size_t)min(eb * 16 + r, E - 1) * d + g * 8;
      f32x4 acc[EB];
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) acc[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // U K steps per trip, all their loads issued before the first MFMA (a
      // load per step behind its own wait made this loop a chain of memory
      // round trips: the DeepSeek-shaped router went 55 -> 43 us); one with 16
      // waves, which split K finer already (two or four measured no faster).
      // d % 8 == 0: an 8-chunk is all in or all out; a lane past d loads its
      // row's first chunk (in bounds) and feeds zeros, as before, so the
      // MFMA sequence and the logits are unchanged.
      constexpr int U = NW >= 16 ? 1 : 4;
      for (int k0 = wv_id * 32; k0 < d; k0 += 32 * NW * U) {
        u32x4 av[U], bv[U][EB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int kk = k0 + u * 32 * NW;
          const int kc = (kk + g * 8) < d ? kk : -g * 8;
          av[u] = *(const u32x4*)(xr + kc);
#pragma unroll
          for (int eb = 0; eb < EB; ++eb) bv[u][eb] = *(const u32x4*)(wr[eb] + kc);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool in = (k0 + u * 32 * NW + g * 8) < d;
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 a = in ? av[u] : z;
#pragma unroll
          for (int eb = 0; eb < EB; ++eb)
            acc[eb] = mfma16(as_bf16x8(a), as_bf16x8(in ? bv[u][eb] : z), acc[eb]);
        }
      }
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) part[wv_id][eb][lane] = acc[eb];
      __syncthreads();
      // sum the wave partials in wave order; C layout of the 16x16 MFMA: lane
      // holds rows 4*(lane/16)+i, column lane%16
      for (int q = tid; q < EB * 64 * 4; q += 64 * NW) {
        const int eb = q / 256, ln = (q >> 2) & 63, i = q & 3;
        float s = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += part[ww][eb][ln][i];
        const int tr = 4 * (ln >> 4) + i, e = eb * 16 + (ln & 15);
        if (e < E) lt[tr][e] = s + (bias ? bias[e] : 0.0f);
      }
    } else {
      const float* x = (const float*)xv;
      const float* w = (const float*)wv;
      for (int p = tid; p < kTokPerWave * E; p += 64 * NW) {
        const int tr = p / E, e = p % E;
        const int tok = min(t0 + tr, T - 1);
        const float s = dot_f32(x + (size_t)tok * d, w + (size_t)e * d, d);
        lt[tr][e] = s + (bias ? bias[e] : 0.0f);
      }
    }
    __syncthreads();
    for (int p = tid; p < kTokPerWave * E; p += 64 * NW) {
      const int tr = p / E, e = p % E;
      if (t0 + tr < T) logits[(size_t)(t0 + tr) * E + e] = lt[tr][e];
    }
  } else {
    for (int p = tid; p < kTokPerWave * E; p += 64 * NW) {
      const int tr = p / E, e = p % E;
      lt[tr][e] = (t0 + tr < T) ? logits[(size_t)(t0 + tr) * E + e] : 0.0f;
    }
  }
  __syncthreads();

  // ---- exact top-k, one token per segment of `seg` lanes ----
  if (seg == 64) {
    // a whole wave per token: radix select of the k-th largest key from
    // ballots (the keys of valid lanes are distinct and above 0; only bits
    // 63..32 and 5..0 can be set), then each winner's rank among the winners
    // from k broadcast keys -- no cross-lane shuffles in a dependent chain
    for (int tr = wv_id; tr < kTokPerWave; tr += NW) {
      const int t = t0 + tr;
      if (t >= T) break;  // uniform
      const unsigned long long key =
          lane < E ? ((unsigned long long)order_key(lt[tr][lane]) << 32) | (uint32_t)(63 - lane) : 0ull;
      unsigned long long th = 0ull;
      auto probe = [&](int b) {
        const unsigned long long c = th | (1ull << b);
        if (__popcll(__ballot(key >= c)) >= k) th = c;
      };
      for (int b = 63; b >= 32; --b) probe(b);
      for (int b = 5; b >= 0; --b) probe(b);
      const bool win = key >= th;  // exactly k lanes
      const uint32_t khi = (uint32_t)(key >> 32), klo = (uint32_t)key;
      int rank = 0;
      for (unsigned long long rest = __ballot(win); rest; rest &= rest - 1ull) {
        const int l = __builtin_ctzll(rest);
        const unsigned long long kl =
            ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)khi, l) << 32) |
            (uint32_t)__builtin_amdgcn_readlane((int)klo, l);
        rank += kl > key ? 1 : 0;
      }
      // weights in slot order (slot 0 the largest), as below
      float lmax = 0.0f, sum = 0.0f, mine = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int l = __builtin_ctzll(__ballot(win && rank == j));
        const float v = order_key_inv((uint32_t)__builtin_amdgcn_readlane((int)khi, l));
        if (j == 0) lmax = v;
        const float w = expf(v - lmax);
        sum += w;
        if (win && rank == j) mine = w;
      }
      if (win) {
        idx[(size_t)t * k + rank] = lane;
        if (gate) gate[(size_t)t * k + rank] = (k == 1) ? 1.0f : mine / sum;
      }
    }
    return;
  }
  const int per = 64 / seg;
  const int ts = lane / seg, e = lane % seg;
  for (int base = wv_id * per; base < kTokPerWave; base += per * NW) {
    const int tr = base + ts;
    const int t = t0 + tr;
    const bool live = (tr < kTokPerWave) && (t < T);
    unsigned long long key = 0ull;
    if (live && e < E)
      key = ((unsigned long long)order_key(lt[tr][e]) << 32) | (uint32_t)(seg - 1 - e);
    unsigned long long top[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        unsigned long long m = key;
        for (int o = 1; o < seg; o <<= 1) {
          unsigned long long v = shfl_xor_u64(m, o);
          m = v > m ? v : m;
        }
        top[j] = m;
        const int win = seg - 1 - (int)(uint32_t)(m & 0xffffffffull);
        if (e == win) key = 0ull;
      }
    }
    if (live && e < k) {
      const float lmax = order_key_inv((uint32_t)(top[0] >> 32));
      float sum = 0.0f, mine = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k) {
          const float w = expf(order_key_inv((uint32_t)(top[j] >> 32)) - lmax);
          sum += w;
          if (j == e) mine = w;
        }
      }
      unsigned long long me = top[0];
#pragma unroll
      for (int j = 1; j < kMaxTopK; ++j)
        if (j == e) me = top[j];
      idx[(size_t)t * k + e] = seg - 1 - (int)(uint32_t)(me & 0xffffffffull);
      if (gate) gate[(size_t)t * k + e] = (k == 1) ? 1.0f : mine / sum;
    }
  }
}

// ---- small batches: route, top-k and permutation in one workgroup ----------
// For a decode step the three are latency, not work: one workgroup of 16 waves
// computes the logits of up to 16*G tokens (the waves split d as above, each
// covering all G token groups), selects each token's top-k, then builds the
// stable expert-major permutation of the T*k <= 1024 assignments at once:
// per-expert counts with LDS atomics, one wave scans them (offsets, LIS), and
// an assignment's row is its expert's offset + the count of equal experts in
// earlier waves + its rank among equal experts in its own wave (a match built
// from log2(64) ballots).  Ranks are computed, never raced, so the order is the
// stable one.

__device__ __forceinline__ unsigned long long lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane ? ((~0ull) >> (64 - lane)) : 0ull;
}

// lanes of this wave holding the same valid expert id as this lane
__device__ __forceinline__ unsigned long long same_expert(int e, bool valid) {
  unsigned long long m = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 6; ++bit) {
    const bool b = (e >> bit) & 1;
    const unsigned long long bal = __ballot(valid && b);
    m &= b ? bal : ~bal;
  }
  return m;
}

// Router logits of a small batch, split over K.  One workgroup pulls the
// batch's token rows from memory slowly (measured ~25 GB/s for one CU: 19 us of
// GEMM for T = 64, d = 4096), so the GEMM first runs over d / KS blocks: block
// b computes the partial logits of all T tokens over K [b*KS, +KS) (4 waves,
// each taking 32-wide K steps KS/128 apart, 16x16x32 MFMA as above; wave
// partials added in wave order), and the routing workgroup adds the block
// partials in block order, so the logits do not depend on block timing.
template <int EB, int G>
__global__ __launch_bounds__(256) void router_partial_kernel(const u16* __restrict__ x,
                                                            const u16* __restrict__ w, int T, int d,
                                                            int E, int KS, float* __restrict__ part) {
  __shared__ f32x4 red[4][G][EB][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  f32x4 acc[G][EB];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) acc[gi][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int steps = KS / 128;  // 1 or 2
#pragma unroll 2
  for (int j = 0; j < steps; ++j) {
    const int k0 = blockIdx.x * KS + j * 128 + wv * 32 + g * 8;
    u32x4 av[G], bv[EB];
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
      av[gi] = *(const u32x4*)(x + (size_t)min(gi * 16 + r, T - 1) * d + k0);
#pragma unroll
    for (int eb = 0; eb < EB; ++eb)
      bv[eb] = *(const u32x4*)(w + (size_t)min(eb * 16 + r, E - 1) * d + k0);
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int eb = 0; eb < EB; ++eb)
        acc[gi][eb] = mfma16(as_bf16x8(av[gi]), as_bf16x8(bv[eb]), acc[gi][eb]);
  }
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) red[wv][gi][eb][lane] = acc[gi][eb];
  __syncthreads();
  // C layout: lane holds token rows 4*(lane/16)+i of its group, expert lane%16
  for (int q = tid; q < G * EB * 256; q += 256) {
    const int gi = q / (EB * 256), eb = (q / 256) % EB, ln = (q >> 2) & 63, i = q & 3;
    const float v = ((red[0][gi][eb][ln][i] + red[1][gi][eb][ln][i]) + red[2][gi][eb][ln][i]) +
                    red[3][gi][eb][ln][i];
    const int tr = gi * 16 + 4 * (ln >> 4) + i, e = eb * 16 + (ln & 15);
    if (tr < T && e < E) part[((size_t)blockIdx.x * T + tr) * E + e] = v;
  }
}

template <int EB, int G>
__global__ __launch_bounds__(1024) void route_permute_small_kernel(
    const u16* __restrict__ x, const u16* __restrict__ w, const float* __restrict__ bias, int T,
    int d, int E, int k, int seg, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ gate, int logits_given, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_assign,
    int32_t* __restrict__ assign_row, double* __restrict__ lis, const float* __restrict__ lpart,
    int nparts) {
  constexpr int NW = 16, TG = 16 * G;
  __shared__ float lt[TG][kMaxExperts + 1];
  __shared__ f32x4 part[NW][G][EB][64];
  __shared__ int s_idx[TG * kMaxTopK];
  __shared__ int cnt[kMaxExperts], ebase[kMaxExperts];
  __shared__ int wc[NW][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv_id = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (!logits_given && lpart) {
    // partial logits of router_partial_kernel, added in block order; a thread's
    // loads are issued together (16 per round)
    for (int q = tid; q < T * E; q += 64 * NW) {
      const int t = q / E, e = q - t * E;
      float sum = 0.0f;
      for (int b0 = 0; b0 < nparts; b0 += 16) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          v[j] = (b0 + j < nparts) ? lpart[((size_t)(b0 + j) * T + t) * E + e] : 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (b0 + j < nparts) sum += v[j];
      }
      const float l = sum + (bias ? bias[e] : 0.0f);
      lt[t][e] = l;
      logits[q] = l;
    }
  } else if (!logits_given) {
    const int r = lane & 15, g = lane >> 4;
    const u16* xr[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) xr[gi] = x + (size_t)min(gi * 16 + r, T - 1) * d + g * 8;
    const u16* wr[EB];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) wr[eb] = w + (size_t)min(eb * 16 + r, E - 1) * d + g * 8;
    f32x4 acc[G][EB];
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) acc[gi][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // all of a wave's K steps are independent: unrolled, their loads are in flight together
#pragma unroll 8
    for (int k0 = wv_id * 32; k0 < d; k0 += 32 * NW) {
      const bool in = (k0 + g * 8) < d;  // d % 8 == 0: an 8-chunk is all in or all out
      u32x4 av[G], bv[EB];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) av[gi] = in ? *(const u32x4*)(xr[gi] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) bv[eb] = in ? *(const u32x4*)(wr[eb] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int eb = 0; eb < EB; ++eb)
          acc[gi][eb] = mfma16(as_bf16x8(av[gi]), as_bf16x8(bv[eb]), acc[gi][eb]);
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) part[wv_id][gi][eb][lane] = acc[gi][eb];
    __syncthreads();
    // wave partials summed in wave order; C layout of the 16x16 MFMA: lane holds
    // token rows 4*(lane/16)+i of its group, expert column lane%16
    for (int q = tid; q < G * EB * 256; q += 64 * NW) {
      const int gi = q / (EB * 256), eb = (q / 256) % EB, ln = (q >> 2) & 63, i = q & 3;
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) sum += part[ww][gi][eb][ln][i];
      const int tr = gi * 16 + 4 * (ln >> 4) + i, e = eb * 16 + (ln & 15);
      if (e < E) lt[tr][e] = sum + (bias ? bias[e] : 0.0f);
    }
    __syncthreads();
    for (int q = tid; q < T * E; q += 64 * NW) logits[q] = lt[q / E][q % E];
  } else {
    for (int q = tid; q < T * E; q += 64 * NW) lt[q / E][q % E] = logits[q];
  }
  __syncthreads();

  // ---- exact top-k, one token per segment of `seg` lanes (as route_topk_kernel)
  const int per = 64 / seg;
  const int ts = lane / seg, e = lane % seg;
  for (int b0 = wv_id * per; b0 < TG; b0 += per * NW) {
    const int t = b0 + ts;
    const bool live = (ts < per) && (t < T);
    unsigned long long key = 0ull;
    if (live && e < E)
      key = ((unsigned long long)order_key(lt[t][e]) << 32) | (uint32_t)(seg - 1 - e);
    unsigned long long top[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        unsigned long long m = key;
        for (int o = 1; o < seg; o <<= 1) {
          unsigned long long v = shfl_xor_u64(m, o);
          m = v > m ? v : m;
        }
        top[j] = m;
        const int win = seg - 1 - (int)(uint32_t)(m & 0xffffffffull);
        if (e == win) key = 0ull;
      }
    }
    if (live && e < k) {
      const float lmax = order_key_inv((uint32_t)(top[0] >> 32));
      float sum = 0.0f, mine = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k) {
          const float wj = expf(order_key_inv((uint32_t)(top[j] >> 32)) - lmax);
          sum += wj;
          if (j == e) mine = wj;
        }
      }
      unsigned long long me = top[0];
#pragma unroll
      for (int j = 1; j < kMaxTopK; ++j)
        if (j == e) me = top[j];
      const int ex = seg - 1 - (int)(uint32_t)(me & 0xffffffffull);
      idx[(size_t)t * k + e] = ex;
      s_idx[t * k + e] = ex;
      if (gate) gate[(size_t)t * k + e] = (k == 1) ? 1.0f : mine / sum;
    }
  }
  if (tid < kMaxExperts) cnt[tid] = 0;
  __syncthreads();

  // ---- stable expert-major permutation of the n = T*k <= 1024 assignments
  const int n = T * k;
  const bool valid = tid < n;
  const int ea = valid ? s_idx[tid] : 0;
  if (valid) atomicAdd(&cnt[ea], 1);
  __syncthreads();
  if (tid < 64) {  // wave 0: exclusive scan and max over the experts
    const int c = (tid < E) ? cnt[tid] : 0;
    int incl = c;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (tid >= o) incl += v;
    }
    int mx = c;
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
    if (tid < E) {
      counts[tid] = c;
      offsets[tid] = incl - c;
      ebase[tid] = incl - c;
    }
    if (tid == E - 1) offsets[E] = incl;
    if (tid == 0 && lis)
      *lis = (double)((long long)E * mx) / (double)((long long)T * k);
  }
  const unsigned long long m = same_expert(ea, valid);
  const int rank = __popcll(m & lanes_below());
  wc[wv_id][lane] = 0;
  __syncthreads();
  if (valid && rank == 0) wc[wv_id][ea] = __popcll(m);
  __syncthreads();
  if (valid) {
    int row = ebase[ea] + rank;
    for (int ww = 0; ww < wv_id; ++ww) row += wc[ww][ea];
    if (row_assign) row_assign[row] = tid;
    if (assign_row) assign_row[tid] = row;
  }
}

}  // namespace

bool route_permute_small_applies(moe_dtype xdt, int T, int E, int k) {
  const int G = (T + 15) / 16, EB = (E + 15) / 16;
  return xdt == MOE_DT_BF16 && T >= 1 && T <= 64 && G * EB <= 4 && T * k <= 1024;
}

// K per block of the split router GEMM (0: not split, the routing workgroup
// computes the logits itself).  Measured on the layer's routing stage: at
// T = 64, d = 4096 the split pair takes 11 instead of 24 us, at T = 16 about
// 1 us less than the one kernel (12.1-12.5 against 13.3-14.0 us).
static int route_part_ks(int T, int d) {
  (void)T;
  return d % 256 == 0 ? 256 : d % 128 == 0 ? 128 : 0;
}

size_t route_part_bytes(moe_dtype xdt, int T, int d, int E, int k) {
  if (!route_permute_small_applies(xdt, T, E, k)) return 0;
  const int ks = route_part_ks(T, d);
  return ks ? (size_t)(d / ks) * T * E * sizeof(float) : 0;
}

hipError_t launch_route_permute_small(const void* x, const void* w_router, const float* b_router,
                                      int T, int d, int E, int k, float* logits, int32_t* idx,
                                      float* gate, bool logits_given, int32_t* counts,
                                      int32_t* offsets, int32_t* row_assign, int32_t* assign_row,
                                      double* lis, float* part_ws, hipStream_t s) {
  if (!route_permute_small_applies(MOE_DT_BF16, T, E, k)) return hipErrorInvalidValue;
  int seg = 1;
  while (seg < E) seg <<= 1;
  const int G = (T + 15) / 16, EB = (E + 15) / 16;
  const int lg = logits_given ? 1 : 0;
  const u16* X = (const u16*)x;
  const u16* W = (const u16*)w_router;
  // the router GEMM over d / ks blocks first (part_ws holds
  // route_part_bytes(...) bytes); without a buffer the workgroup computes it
  const int ks = route_part_ks(T, d);
  const float* part = (!logits_given && part_ws && ks) ? part_ws : nullptr;
  const int nparts = part ? d / ks : 0;
  if (part) {
#define MOE_RPART(EBV, GV)                                                                      \
  hipLaunchKernelGGL((router_partial_kernel<EBV, GV>), dim3(nparts), dim3(256), 0, s, X, W, T, d, \
                     E, ks, part_ws)
    switch (EB * 8 + G) {
      case 1 * 8 + 1: MOE_RPART(1, 1); break;
      case 1 * 8 + 2: MOE_RPART(1, 2); break;
      case 1 * 8 + 3: MOE_RPART(1, 3); break;
      case 1 * 8 + 4: MOE_RPART(1, 4); break;
      case 2 * 8 + 1: MOE_RPART(2, 1); break;
      case 2 * 8 + 2: MOE_RPART(2, 2); break;
      case 3 * 8 + 1: MOE_RPART(3, 1); break;
      case 4 * 8 + 1: MOE_RPART(4, 1); break;
      default: return hipErrorInvalidValue;
    }
#undef MOE_RPART
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define MOE_RPS(EBV, GV)                                                                         \
  hipLaunchKernelGGL((route_permute_small_kernel<EBV, GV>), dim3(1), dim3(1024), 0, s, X, W,     \
                     b_router, T, d, E, k, seg, logits, idx, gate, lg, counts, offsets,          \
                     row_assign, assign_row, lis, part, nparts)
  switch (EB * 8 + G) {
    case 1 * 8 + 1: MOE_RPS(1, 1); break;
    case 1 * 8 + 2: MOE_RPS(1, 2); break;
    case 1 * 8 + 3: MOE_RPS(1, 3); break;
    case 1 * 8 + 4: MOE_RPS(1, 4); break;
    case 2 * 8 + 1: MOE_RPS(2, 1); break;
    case 2 * 8 + 2: MOE_RPS(2, 2); break;
    case 3 * 8 + 1: MOE_RPS(3, 1); break;
    case 4 * 8 + 1: MOE_RPS(4, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_RPS
  return hipGetLastError();
}

hipError_t launch_route_topk(const void* x, moe_dtype xdt, const void* w_router,
                             const float* b_router, int T, int d, int E, int k, float* logits,
                             int32_t* idx, float* gate, bool logits_given, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int seg = 1;
  while (seg < E) seg <<= 1;
  const int groups = (T + kTokPerWave - 1) / kTokPerWave;
  const dim3 grid(groups);
  const int lg = logits_given ? 1 : 0;
  if (xdt == MOE_DT_F32) {
    hipLaunchKernelGGL((route_topk_kernel<1, 1, true>), grid, dim3(64), 0, s, x, w_router,
                       b_router, T, d, E, k, seg, logits, idx, gate, lg);
    return hipGetLastError();
  }
  // up to 256 token groups (decode, 4096-token prefill): 16 waves share each
  // group's reduction over d; more groups: 4 waves per group fill the chip
  const bool wide = groups <= 256;
  const int eb = (E + 15) / 16;
#define MOE_ROUTE_LAUNCH(EBV, NWV)                                                       \
  hipLaunchKernelGGL((route_topk_kernel<EBV, NWV, false>), grid, dim3(64 * NWV), 0, s, x, \
                     w_router, b_router, T, d, E, k, seg, logits, idx, gate, lg)
  switch (eb) {
    case 1:
      if (wide) MOE_ROUTE_LAUNCH(1, 16); else MOE_ROUTE_LAUNCH(1, 4);
      break;
    case 2:
      if (wide) MOE_ROUTE_LAUNCH(2, 16); else MOE_ROUTE_LAUNCH(2, 4);
      break;
    case 3:
      if (wide) MOE_ROUTE_LAUNCH(3, 16); else MOE_ROUTE_LAUNCH(3, 4);
      break;
    default:
      if (wide) MOE_ROUTE_LAUNCH(4, 16); else MOE_ROUTE_LAUNCH(4, 4);
      break;
  }
#undef MOE_ROUTE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
