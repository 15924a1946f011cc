// atomic.hip -- routing and expert-centric grouping of atomic experts on a
// Cartesian router grid.
//
// "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale" -- What
// carries the argument: an expert id is a cell (i, j) of an nr x nc grid, scored
// as the sum of a row and a column log-probability (Eq. 8); each token keeps its
// exact top-K cells (Axiom ledger: the merge-selection recovers the exact global
// top-K); expert-centric scheduling groups the kept (token, expert) pairs by
// expert.
//
//   log_softmax_kernel   row / column log-probabilities from the router logits
//   grid_topk_kernel     per token: sort the column scores, binary-search the
//                        K-th largest cell score over fp32 keys (each count is
//                        one binary search per row in the sorted columns), then
//                        one pass over the grid in id order writes the kept ids
//                        (ascending), their softmax gates and a kept-cell bitmap
//   grid_count/.../rows_kernel
//                        counting sort of the kept pairs by expert from the
//                        bitmap: per (32-expert word, 64-token chunk) counts,
//                        per-expert offsets, then each expert's rows in token
//                        order -- deterministic, no atomics
// Cells with equal fp32 scores are ordered by id, so the selection is unique.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGridMax = 1024;   // nr, nc limit
constexpr int kPermChunkT = 64;  // tokens per counting chunk
constexpr int kRowsTok = 256;    // tokens staged per round of grid_rows_kernel
constexpr int kRowsSpan = 1024;  // tokens per grid_rows_kernel block (a multiple of both)
constexpr int kTopkWideMaxT = 64;  // up to this many tokens: 1024-thread top-K blocks

__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// the float whose key is k (for keys of non-NaN floats: s >= kf(k) <=> fkey(s) >= k,
// with -0.0 and +0.0 equal on both sides)
__device__ __forceinline__ float kf(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int wave_sum(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// block (256 threads) sum; every thread gets the total
template <int NW = 4>
__device__ __forceinline__ int block_sum(int v, int* red) {
  const int tid = threadIdx.x;
  v = wave_sum(v);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  int s = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) s += red[i];
  return s;
}

// exclusive scan of one value per thread over the block (NW waves); the
// block total goes to *total
template <int NW = 4>
__device__ __forceinline__ int block_exscan(int v, int* red, int* total = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  __syncthreads();
  if (lane == 63) red[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += red[i];
  if (total) {
    int s = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) s += red[i];
    *total = s;
  }
  return base + incl - v;
}

// ---- log-probabilities ---------------------------------------------------------
// one 256-thread block per token; the logits may arrive as NS partial sums (K
// slices of the router GEMM, split_stride floats apart), added here in slice
// order.  A thread's NS loads of an element are all issued before the adds (the
// partial sums come from another launch, so each load is a full memory round
// trip; a runtime-length loop waited for each in turn).
constexpr int kLsThreads = 256;

template <int NS>
__global__ __launch_bounds__(kLsThreads) void log_softmax_kernel(const float* __restrict__ l,
                                                                 int n, size_t split_stride,
                                                                 float* __restrict__ out) {
  __shared__ float row[kGridMax];
  __shared__ float red[kLsThreads / 64];
  const float* r = l + (size_t)blockIdx.x * n;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float m = -INFINITY;
  for (int i = tid; i < n; i += kLsThreads) {
    float p[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) p[q] = r[(size_t)q * split_stride + i];
    float v = p[0];
#pragma unroll
    for (int q = 1; q < NS; ++q) v += p[q];
    row[i] = v;
    m = fmaxf(m, v);
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) red[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();  // red is reused below
  float sum = 0.0f;
  for (int i = tid; i < n; i += kLsThreads) sum += expf(row[i] - m);  // this thread's own elements
  sum = wave_sum_f(sum);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  const float lse = m + logf(((red[0] + red[1]) + red[2]) + red[3]);
  for (int i = tid; i < n; i += kLsThreads) out[(size_t)blockIdx.x * n + i] = row[i] - lse;
}

// ---- exact top-K over the grid -----------------------------------------------
// The column scores are sorted once (descending, ties by column id); for a row i
// the cells at or above any key form a prefix of that order, found by binary
// search, so theta (the K-th largest key) comes from a binary search over the
// 32-bit keys with one such count per row.  Emission then walks the grid in
// rounds of NT consecutive 32-cell words (one word per thread): a cell is kept
// if its key is above theta, or equal to it while the ties before it (in id
// order, a block scan per round) are fewer than the ties needed; positions come
// from a block scan of the kept counts, so ids and gates leave in ascending id
// order and the bitmap words and their prefixes in coalesced stores.
// NT threads per block: 256 when many tokens fill the chip, 1024 at decode
// sizes, where each token's block is alone on its CU and the search and the
// walk over the grid are its latency
template <int NT>
__global__ __launch_bounds__(NT) void grid_topk_kernel(const float* __restrict__ pr,
                                                        const float* __restrict__ pc, int nr,
                                                        int nc, int K, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate,
                                                        uint32_t* __restrict__ bits,
                                                        int32_t* __restrict__ bitpre) {
  __shared__ float a[kGridMax], b[kGridMax], bv[kGridMax];
  __shared__ unsigned long long bk[kGridMax];  // sort keys: fkey(b) << 32 | ~column
  constexpr int NW = NT / 64;
  __shared__ int red[NW];
  __shared__ float redf[NW];
  const int t = blockIdx.x, tid = threadIdx.x;
  int ncp = 1;
  while (ncp < nc) ncp <<= 1;
  for (int i = tid; i < nr; i += NT) a[i] = pr[(size_t)t * nr + i];
  for (int j = tid; j < ncp; j += NT) {
    unsigned long long key = 0ull;  // padding sorts last
    if (j < nc) {
      const float v = pc[(size_t)t * nc + j];
      b[j] = v;
      key = ((unsigned long long)fkey(v) << 32) | (uint32_t)(~(uint32_t)j);
    }
    bk[j] = key;
  }
  __syncthreads();
  // bitonic sort of bk, descending
  for (int size = 2; size <= ncp; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int q = tid; q < ncp / 2; q += NT) {
        const int lo = 2 * q - (q & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const unsigned long long x = bk[lo], y = bk[hi];
        if (desc ? (x < y) : (x > y)) {
          bk[lo] = y;
          bk[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < nc; j += NT) bv[j] = b[~(uint32_t)bk[j]];
  __syncthreads();
  auto count_ge = [&](uint32_t kt) {
    const float th = kf(kt);
    int c = 0;
    for (int i = tid; i < nr; i += NT) {
      const float ai = a[i];
      int lo = 0, hi = nc;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ai + bv[mid] >= th)
          lo = mid + 1;
        else
          hi = mid;
      }
      c += lo;
    }
    return block_sum<NW>(c, red);
  };
  // the largest and smallest cell scores: row extreme plus column extreme
  float am = -INFINITY, an = INFINITY;
  for (int i = tid; i < nr; i += NT) {
    am = fmaxf(am, a[i]);
    an = fminf(an, a[i]);
  }
  for (int o = 32; o > 0; o >>= 1) {
    am = fmaxf(am, __shfl_xor(am, o, 64));
    an = fminf(an, __shfl_xor(an, o, 64));
  }
  __shared__ float redn[NW];
  if ((tid & 63) == 0) {
    redf[tid >> 6] = am;
    redn[tid >> 6] = an;
  }
  __syncthreads();
  float rmax = redf[0], rmin = redn[0];
#pragma unroll
  for (int q = 1; q < NW; ++q) {
    rmax = fmaxf(rmax, redf[q]);
    rmin = fminf(rmin, redn[q]);
  }
  const float smax = rmax + bv[0];
  const float smin = rmin + bv[nc - 1];
  // theta: the largest key with at least K cells at or above it.  A probe with
  // exactly K cells at or above it ends the search early: those cells are the
  // selection (kept: key >= probe, no ties to break).
  // Per row i of this thread (i = tid + NT*s), the count of its cells at or
  // above a key is a prefix length of the sorted column order; the search keeps
  // that length at lo (rub) and at the last probe that fell short (rlb) and
  // looks for the next probe's length only between them.
  uint32_t lo = fkey(smin), hi = fkey(smax);
  int c_lo = nr * nc;  // cells at or above key lo
  constexpr int kRowsPer = kGridMax / NT;
  int rlb[kRowsPer], rub[kRowsPer], rl[kRowsPer];
#pragma unroll
  for (int s = 0; s < kRowsPer; ++s) {
    rlb[s] = 0;
    rub[s] = nc;
  }
  while (lo < hi) {
    const uint32_t mid = lo + (uint32_t)(((uint64_t)hi - lo + 1) >> 1);
    const float th = kf(mid);
    int cpart = 0;
#pragma unroll
    for (int s = 0; s < kRowsPer; ++s) {
      const int i = tid + NT * s;
      rl[s] = 0;
      if (i < nr) {
        const float ai = a[i];
        int l = rlb[s], h = rub[s];
        while (l < h) {
          const int m = (l + h) >> 1;
          if (ai + bv[m] >= th)
            l = m + 1;
          else
            h = m;
        }
        rl[s] = l;
        cpart += l;
      }
    }
    const int c = block_sum<NW>(cpart, red);
    if (c >= K) {
      lo = mid;
      c_lo = c;
#pragma unroll
      for (int s = 0; s < kRowsPer; ++s) rub[s] = rl[s];
      if (c == K) break;
    } else {
      hi = mid - 1;
#pragma unroll
      for (int s = 0; s < kRowsPer; ++s) rlb[s] = rl[s];
    }
  }
  const uint32_t theta = lo;
  // exactly K cells at or above theta (the usual case): they are the selection;
  // otherwise theta is the K-th largest key and ties at it are broken by id
  const bool exact = c_lo == K;
  const int c_gt = exact ? K : (theta == 0xffffffffu ? 0 : count_ge(theta + 1u));
  const int m_tie = K - c_gt;  // cells at theta to keep, lowest ids first
  const float thf = kf(theta);

  const int W = nr * nc / 32, nw = nc / 32;
  int base = 0, ties = 0;
  float wsum = 0.0f;
  int32_t* out = idx + (size_t)t * K;
  float* gout = gate + (size_t)t * K;
  for (int w0 = 0; w0 < W; w0 += NT) {
    const int w = w0 + tid;
    uint32_t word = 0u;
    int i = 0, j0 = 0;
    if (exact) {  // block-uniform: keep every cell at or above theta
      if (w < W) {
        i = w / nw;
        j0 = (w - i * nw) * 32;
        const float ai = a[i];
        for (int q0 = 0; q0 < 32; ++q0) {
          const int q = (q0 + tid) & 31;  // rotated per lane: no LDS bank conflicts
          word |= (uint32_t)(ai + b[j0 + q] >= thf) << q;
        }
      }
    } else {
      uint32_t tiew = 0u;
      if (w < W) {
        i = w / nw;
        j0 = (w - i * nw) * 32;
        const float ai = a[i];
        for (int q0 = 0; q0 < 32; ++q0) {
          const int q = (q0 + tid) & 31;
          const float sv = ai + b[j0 + q];
          word |= (uint32_t)(sv > thf) << q;
          tiew |= (uint32_t)(sv == thf) << q;
        }
      }
      // ties before this word in id order, then keep as many as are still needed
      const int nt = __popc(tiew);
      int tsum;
      const int tb = ties + block_exscan<NW>(nt, red, &tsum);
      int room = min(max(m_tie - tb, 0), nt);
      while (room > 0) {  // lowest tie columns first
        const uint32_t low = tiew & (0u - tiew);
        word |= low;
        tiew ^= low;
        --room;
      }
      ties += tsum;
    }
    const int nk = __popc(word);
    int ksum;
    const int pos = base + block_exscan<NW>(nk, red, &ksum);
    if (w < W) {
      bits[(size_t)t * W + w] = word;
      bitpre[(size_t)t * W + w] = pos;
      int p = pos;
      uint32_t ww = word;
      const float ai = a[i];
      while (ww && p < K) {  // p < K always holds for finite scores
        const int q = __ffs(ww) - 1;
        ww &= ww - 1u;
        const float wv = expf((ai + b[j0 + q]) - smax);
        out[p] = i * nc + j0 + q;
        gout[p] = wv;
        wsum += wv;
        ++p;
      }
    }
    base += ksum;
  }
  // normalise: total over the block in a fixed order
  wsum = wave_sum_f(wsum);
  __syncthreads();
  if ((tid & 63) == 0) redf[tid >> 6] = wsum;
  __syncthreads();
  // pairwise in wave order (NW = 4: (0 + 1) + (2 + 3))
  float part[NW];
#pragma unroll
  for (int q = 0; q < NW; ++q) part[q] = redf[q];
#pragma unroll
  for (int h = 1; h < NW; h <<= 1)
#pragma unroll
    for (int q = 0; q + h < NW; q += 2 * h) part[q] = part[q] + part[q + h];
  const float total = part[0];
  for (int p = tid; p < K; p += NT) gout[p] = gout[p] / total;
}

// ---- counting sort of the kept pairs by expert ---------------------------------
// thread = (32-expert word wc, token chunk c): per-bit counts of the chunk,
// kept bit-sliced while the chunk's words are added (plane p holds bit p of
// all 32 counts; a count never exceeds kPermChunkT = 64, so 7 planes), then
// unpacked once; the chunk's loads are unrolled so many are in flight
__global__ __launch_bounds__(256) void grid_count_kernel(const uint32_t* __restrict__ bits, int T,
                                                         int W, int32_t* __restrict__ ccount) {
  static_assert(kPermChunkT <= 127, "7 count planes");
  const int wc = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  if (wc >= W) return;
  uint32_t plane[7] = {0u, 0u, 0u, 0u, 0u, 0u, 0u};
  const int t1 = min((c + 1) * kPermChunkT, T);
#pragma unroll 16
  for (int t = c * kPermChunkT; t < t1; ++t) {
    uint32_t carry = bits[(size_t)t * W + wc];
#pragma unroll
    for (int p = 0; p < 7; ++p) {
      const uint32_t nc = plane[p] & carry;
      plane[p] ^= carry;
      carry = nc;
    }
  }
  int32_t* o = ccount + (size_t)c * W * 32 + (size_t)wc * 32;
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    int v = 0;
#pragma unroll
    for (int p = 0; p < 7; ++p) v |= (int)((plane[p] >> q) & 1u) << p;
    o[q] = v;
  }
}

// thread per expert: counts (sum over chunks) and the chunk prefixes, in place
__global__ __launch_bounds__(256) void grid_chunkprefix_kernel(int32_t* __restrict__ ccount,
                                                               int nchunk, int N,
                                                               int32_t* __restrict__ counts) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  // loads of 16 chunks are issued before their prefixes are written
  int run = 0;
  int c0 = 0;
  for (; c0 + 16 <= nchunk; c0 += 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = ccount[(size_t)(c0 + u) * N + n];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      ccount[(size_t)(c0 + u) * N + n] = run;
      run += v[u];
    }
  }
  for (int c = c0; c < nchunk; ++c) {
    int32_t* p = ccount + (size_t)c * N + n;
    const int v = *p;
    *p = run;
    run += v;
  }
  counts[n] = run;
}

// exclusive offsets over the experts and LIS, in three launches: per-block
// (256 experts) sums and maxima, one block scanning those, then each expert's
// offset = its block's prefix + its rank inside the block
__global__ __launch_bounds__(256) void grid_blocksum_kernel(const int32_t* __restrict__ counts,
                                                            int N, int32_t* __restrict__ bsum,
                                                            int32_t* __restrict__ bmax) {
  __shared__ int red[4];
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int v = n < N ? counts[n] : 0;
  int m = v;
  for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
  const int tot = block_sum(v, red);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    bsum[blockIdx.x] = tot;
    bmax[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
  }
}

__global__ __launch_bounds__(1024) void grid_blockscan_kernel(int32_t* __restrict__ bsum,
                                                              const int32_t* __restrict__ bmax,
                                                              int nb, int N, int T, int K,
                                                              int32_t* __restrict__ offsets,
                                                              double* __restrict__ lis) {
  __shared__ int part[1024];
  __shared__ int mx[1024];
  const int tid = threadIdx.x;
  const int per = (nb + 1023) / 1024;
  const int b0 = min(tid * per, nb), b1 = min(b0 + per, nb);
  int sum = 0, best = 0;
  for (int b = b0; b < b1; ++b) {
    sum += bsum[b];
    best = max(best, bmax[b]);
  }
  part[tid] = sum;
  mx[tid] = best;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  for (int o = 512; o > 0; o >>= 1) {
    if (tid < o) mx[tid] = max(mx[tid], mx[tid + o]);
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int b = b0; b < b1; ++b) {  // in place: block sums become block prefixes
    const int v = bsum[b];
    bsum[b] = run;
    run += v;
  }
  if (tid == 1023) offsets[N] = part[1023];
  if (tid == 0) *lis = T == 0 ? NAN : (double)((int64_t)N * mx[0]) / (double)((int64_t)T * K);
}

__global__ __launch_bounds__(256) void grid_offsets_kernel(const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ bpre, int N,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int red[4];
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int v = n < N ? counts[n] : 0;
  const int r = block_exscan(v, red);
  if (n < N) offsets[n] = bpre[blockIdx.x] + r;
}

// Block: 256 experts (8 bitmap words) x one range of kRowsSpan tokens; thread:
// one expert, which writes its rows of row_assign for those tokens in token
// order, from its offset plus the chunk prefix at the range's start on.
// Tokens are staged kRowsTok at a time (words and prefixes of the block's 8
// words; the next round's loads are issued before this round is processed);
// per 32 tokens the thread gathers its bit of each into a mask and walks the
// set bits.  The slots of one token that the 64 experts of a wave keep are
// consecutive, so assign_row stores from a wave land together too.
__global__ __launch_bounds__(256) void grid_rows_kernel(const uint32_t* __restrict__ bits,
                                                        const int32_t* __restrict__ bitpre, int T,
                                                        int W, int K,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ cpre,
                                                        int32_t* __restrict__ row_assign,
                                                        int32_t* __restrict__ assign_row) {
  __shared__ uint32_t sw[kRowsTok][8];
  __shared__ int32_t sp[kRowsTok][8];
  const int tid = threadIdx.x;
  const int wc0 = blockIdx.x * 8;
  const int N = W * 32;
  const int n = blockIdx.x * 256 + tid;
  const int myw = tid >> 5, b = tid & 31;
  const uint32_t below = (1u << b) - 1u;
  const int tbeg = blockIdx.y * kRowsSpan, tend = min(tbeg + kRowsSpan, T);
  int row = n < N ? offsets[n] + cpre[(size_t)(tbeg / kPermChunkT) * N + n] : 0;
  uint32_t rw[8];
  int rp[8];
  auto load = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i;
      const int t = t0 + (q >> 3), w = wc0 + (q & 7);
      const bool in = t < tend && w < W;
      rw[i] = in ? bits[(size_t)t * W + w] : 0u;
      rp[i] = in ? bitpre[(size_t)t * W + w] : 0;
    }
  };
  load(tbeg);
  for (int t0 = tbeg; t0 < tend; t0 += kRowsTok) {
    __syncthreads();  // the previous round's reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i;
      sw[q >> 3][q & 7] = rw[i];
      sp[q >> 3][q & 7] = rp[i];
    }
    __syncthreads();
    if (t0 + kRowsTok < tend) load(t0 + kRowsTok);
    if (n >= N) continue;
    for (int u0 = 0; u0 < kRowsTok; u0 += 32) {
      uint32_t m = 0u;  // bit u: token t0 + u0 + u keeps expert n
#pragma unroll
      for (int u = 0; u < 32; ++u) m |= ((sw[u0 + u][myw] >> b) & 1u) << u;
      while (m) {
        const int u = u0 + __ffs(m) - 1;
        m &= m - 1u;
        const uint32_t w = sw[u][myw];
        const int a = (t0 + u) * K + sp[u][myw] + __popc(w & below);
        if (row_assign) row_assign[row] = a;
        if (assign_row) assign_row[a] = row;
        ++row;
      }
    }
  }
}

__global__ void iota_kernel(int32_t* out, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = i;
}

__global__ void iota_kernel_zero(int32_t* out, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = 0;
}

}  // namespace

hipError_t launch_log_softmax_rows(const float* l, int T, int n, float* out, hipStream_t s,
                                   int nsplit, size_t split_stride) {
  if (T == 0) return hipSuccess;
  if (n > kGridMax) return hipErrorInvalidValue;
  const dim3 grid((unsigned)T), block(kLsThreads);
  switch (nsplit) {
    case 1: hipLaunchKernelGGL(log_softmax_kernel<1>, grid, block, 0, s, l, n, split_stride, out); break;
    case 2: hipLaunchKernelGGL(log_softmax_kernel<2>, grid, block, 0, s, l, n, split_stride, out); break;
    case 4: hipLaunchKernelGGL(log_softmax_kernel<4>, grid, block, 0, s, l, n, split_stride, out); break;
    case 8: hipLaunchKernelGGL(log_softmax_kernel<8>, grid, block, 0, s, l, n, split_stride, out); break;
    case 16: hipLaunchKernelGGL(log_softmax_kernel<16>, grid, block, 0, s, l, n, split_stride, out); break;
    default: return hipErrorInvalidValue;  // the router GEMM splits are powers of two up to 16
  }
  return hipGetLastError();
}

hipError_t launch_grid_topk(const float* pr, const float* pc, int T, int nr, int nc, int K,
                            int32_t* idx, float* gate, uint32_t* bits, int32_t* bitpre,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (nr > kGridMax || nc > kGridMax || nc % 32 != 0) return hipErrorInvalidValue;
if (T <= kTopkWideMaxT)
    hipLaunchKernelGGL(grid_topk_kernel<1024>, dim3(T), dim3(1024), 0, s, pr, pc, nr, nc, K, idx, gate,
                     bits, bitpre);
  else
    hipLaunchKernelGGL(grid_topk_kernel<256>, dim3(T), dim3(256), 0, s, pr, pc, nr, nc, K, idx, gate,
                     bits, bitpre);
  return hipGetLastError();
}

size_t grid_permute_ws_bytes(int T, int N) {
  const size_t nchunk = (size_t)(T + kPermChunkT - 1) / kPermChunkT;
  const size_t nb = (size_t)(N + 255) / 256;
  return (nchunk * (size_t)N + 2 * nb) * sizeof(int32_t);
}

hipError_t launch_grid_permute(const uint32_t* bits, const int32_t* bitpre, int T, int N, int K,
                               int32_t* counts, int32_t* offsets, int32_t* row_assign,
                               int32_t* assign_row, double* lis, void* ws, hipStream_t s) {
  if (N % 32 != 0) return hipErrorInvalidValue;
  const int W = N / 32;
  const int nchunk = (T + kPermChunkT - 1) / kPermChunkT;
  int32_t* ccount = (int32_t*)ws;
  if (T > 0) {
    const dim3 grid((unsigned)((W + 255) / 256), (unsigned)nchunk);
    hipLaunchKernelGGL(grid_count_kernel, grid, dim3(256), 0, s, bits, T, W, ccount);
  }
  if (T > 0)
    hipLaunchKernelGGL(grid_chunkprefix_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s,
                       ccount, nchunk, N, counts);
  else
    hipLaunchKernelGGL(iota_kernel_zero, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s,
                       counts, N);
  const int nb = (N + 255) / 256;
  int32_t* bsum = ccount + (size_t)nchunk * N;
  int32_t* bmax = bsum + nb;
  hipLaunchKernelGGL(grid_blocksum_kernel, dim3((unsigned)nb), dim3(256), 0, s, counts, N, bsum,
                     bmax);
  hipLaunchKernelGGL(grid_blockscan_kernel, dim3(1), dim3(1024), 0, s, bsum, bmax, nb, N, T, K,
                     offsets, lis);
  hipLaunchKernelGGL(grid_offsets_kernel, dim3((unsigned)nb), dim3(256), 0, s, counts, bsum, N,
                     offsets);
  if (T > 0 && (row_assign || assign_row))
    hipLaunchKernelGGL(grid_rows_kernel,
                       dim3((unsigned)((W + 7) / 8), (unsigned)((T + kRowsSpan - 1) / kRowsSpan)),
                       dim3(256), 0, s, bits, bitpre, T, W, K, offsets, ccount, row_assign,
                       assign_row);
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* out, int n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(iota_kernel, dim3((n + 255) / 256), dim3(256), 0, s, out, n);
  return hipGetLastError();
}

}  // namespace moe
