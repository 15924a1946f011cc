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
      for (int k0 = wv_id * 32; k0 < d; k0 += 32 * NW) {
        const bool in = (k0 + g * 8) < d;  // d % 8 == 0: an 8-chunk is all in or all out
        u32x4 av = in ? *(const u32x4*)(xr + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
          u32x4 bv = in ? *(const u32x4*)(wr[eb] + k0) : u32x4{0, 0, 0, 0};
          acc[eb] = mfma16(as_bf16x8(av), as_bf16x8(bv), acc[eb]);
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
        const float* xr = x + (size_t)tok * d;
        const float* wr = w + (size_t)e * d;
        float s = 0.0f;
        for (int i = 0; i < d; ++i) s = fmaf(xr[i], wr[i], s);
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

}  // namespace

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
