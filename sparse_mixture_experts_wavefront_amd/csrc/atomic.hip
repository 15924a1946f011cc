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
//   grid_count/scan/write_kernel
//                        counting sort of the kept pairs by expert from the
//                        bitmap: per (32-expert word, 256-token chunk) counts,
//                        per-expert offsets, then rows in token order inside
//                        each expert -- deterministic, no atomics
// Cells with equal fp32 scores are ordered by id, so the selection is unique.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGridMax = 1024;   // nr, nc limit
constexpr int kPermChunkT = 256; // tokens per counting chunk

__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
__device__ __forceinline__ int block_sum(int v, int* red) {
  const int tid = threadIdx.x;
  v = wave_sum(v);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// exclusive scan of one value per thread over the block (256 threads)
__device__ __forceinline__ int block_exscan(int v, int* red) {
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
  return base + incl - v;
}

// ---- log-probabilities ---------------------------------------------------------
__global__ __launch_bounds__(64) void log_softmax_kernel(const float* __restrict__ l, int n,
                                                         float* __restrict__ out) {
  const float* r = l + (size_t)blockIdx.x * n;
  float m = -INFINITY;
  for (int i = threadIdx.x; i < n; i += 64) m = fmaxf(m, r[i]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float s = 0.0f;
  for (int i = threadIdx.x; i < n; i += 64) s += expf(r[i] - m);
  s = wave_sum_f(s);
  const float lse = m + logf(s);
  for (int i = threadIdx.x; i < n; i += 64) out[(size_t)blockIdx.x * n + i] = r[i] - lse;
}

// ---- exact top-K over the grid -----------------------------------------------
__global__ __launch_bounds__(256) void grid_topk_kernel(const float* __restrict__ pr,
                                                        const float* __restrict__ pc, int nr,
                                                        int nc, int K, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate,
                                                        uint32_t* __restrict__ bits,
                                                        int32_t* __restrict__ bitpre) {
  __shared__ float a[kGridMax], b[kGridMax], bs[kGridMax];
  __shared__ int red[4];
  __shared__ float redf[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  int ncp = 1;
  while (ncp < nc) ncp <<= 1;
  for (int i = tid; i < nr; i += 256) a[i] = pr[(size_t)t * nr + i];
  for (int j = tid; j < ncp; j += 256) {
    const float v = j < nc ? pc[(size_t)t * nc + j] : -INFINITY;
    if (j < nc) b[j] = v;
    bs[j] = v;
  }
  __syncthreads();
  // bitonic sort of bs, descending
  for (int size = 2; size <= ncp; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int q = tid; q < ncp / 2; q += 256) {
        const int lo = 2 * q - (q & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const float x = bs[lo], y = bs[hi];
        if (desc ? (x < y) : (x > y)) {
          bs[lo] = y;
          bs[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  // cells with key >= kt: per row, the columns form a prefix of bs
  auto count_ge = [&](uint32_t kt) {
    int c = 0;
    for (int i = tid; i < nr; i += 256) {
      int lo = 0, hi = nc;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (fkey(a[i] + bs[mid]) >= kt)
          lo = mid + 1;
        else
          hi = mid;
      }
      c += lo;
    }
    return block_sum(c, red);
  };
  // theta: the largest key with at least K cells at or above it
  uint32_t lo = 0u, hi = 0xffffffffu;
  while (lo < hi) {
    const uint32_t mid = lo + (uint32_t)(((uint64_t)hi - lo + 1) >> 1);
    if (count_ge(mid) >= K)
      lo = mid;
    else
      hi = mid - 1;
  }
  const uint32_t theta = lo;
  const int c_gt = theta == 0xffffffffu ? 0 : count_ge(theta + 1);
  const int m_tie = K - c_gt;  // cells at theta to keep, lowest ids first

  // rows in id order: thread tid owns rows [r0, r1)
  const int rpt = (nr + 255) / 256;
  const int r0 = min(tid * rpt, nr), r1 = min(r0 + rpt, nr);
  int gt_sum = 0, eq_sum = 0;
  for (int i = r0; i < r1; ++i)
    for (int j = 0; j < nc; ++j) {
      const uint32_t kk = fkey(a[i] + b[j]);
      gt_sum += kk > theta;
      eq_sum += kk == theta;
    }
  const int eq_before = block_exscan(eq_sum, red);
  int take = min(max(m_tie - eq_before, 0), eq_sum);  // ties this thread keeps
  const int pos0 = block_exscan(gt_sum + take, red);
  // max score (the row max plus the column max) for the softmax
  float am = -INFINITY;
  for (int i = tid; i < nr; i += 256) am = fmaxf(am, a[i]);
  for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  __syncthreads();
  if ((tid & 63) == 0) redf[tid >> 6] = am;
  __syncthreads();
  const float smax = fmaxf(fmaxf(redf[0], redf[1]), fmaxf(redf[2], redf[3])) + bs[0];

  const int W = nr * nc / 32;
  int pos = pos0;
  float wsum = 0.0f;
  int32_t* out = idx + (size_t)t * K;
  float* gout = gate + (size_t)t * K;
  for (int i = r0; i < r1; ++i) {
    for (int w0 = 0; w0 < nc; w0 += 32) {
      uint32_t word = 0u;
      const int wpre = pos;  // kept cells of the token before this word
      for (int jj = 0; jj < 32; ++jj) {
        const int j = w0 + jj;
        const float sv = a[i] + b[j];
        const uint32_t kk = fkey(sv);
        bool keep = kk > theta;
        if (!keep && kk == theta && take > 0) {
          keep = true;
          --take;
        }
        if (keep) {
          word |= 1u << jj;
          const float wv = expf(sv - smax);
          out[pos] = i * nc + j;
          gout[pos] = wv;
          wsum += wv;
          ++pos;
        }
      }
      const size_t wi = (size_t)t * W + (size_t)(i * nc + w0) / 32;
      bits[wi] = word;
      bitpre[wi] = wpre;
    }
  }
  // normalise: total over the block in a fixed order
  wsum = wave_sum_f(wsum);
  __syncthreads();
  if ((tid & 63) == 0) redf[tid >> 6] = wsum;
  __syncthreads();
  const float total = (redf[0] + redf[1]) + (redf[2] + redf[3]);
  for (int p = pos0; p < pos; ++p) gout[p] = gout[p] / total;
}

// ---- counting sort of the kept pairs by expert ---------------------------------
// thread = (32-expert word wc, token chunk c): per-bit counts of the chunk
__global__ __launch_bounds__(256) void grid_count_kernel(const uint32_t* __restrict__ bits, int T,
                                                         int W, int32_t* __restrict__ ccount) {
  const int wc = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  if (wc >= W) return;
  int cnt[32];
#pragma unroll
  for (int q = 0; q < 32; ++q) cnt[q] = 0;
  const int t1 = min((c + 1) * kPermChunkT, T);
  for (int t = c * kPermChunkT; t < t1; ++t) {
    const uint32_t w = bits[(size_t)t * W + wc];
    if (w) {
#pragma unroll
      for (int q = 0; q < 32; ++q) cnt[q] += (w >> q) & 1u;
    }
  }
  int32_t* o = ccount + (size_t)c * W * 32 + (size_t)wc * 32;
#pragma unroll
  for (int q = 0; q < 32; ++q) o[q] = cnt[q];
}

// thread per expert: counts (sum over chunks) and the chunk prefixes, in place
__global__ __launch_bounds__(256) void grid_chunkprefix_kernel(int32_t* __restrict__ ccount,
                                                               int nchunk, int N,
                                                               int32_t* __restrict__ counts) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  int run = 0;
  for (int c = 0; c < nchunk; ++c) {
    int32_t* p = ccount + (size_t)c * N + n;
    const int v = *p;
    *p = run;
    run += v;
  }
  counts[n] = run;
}

// one block of 1024 threads: exclusive offsets over the experts and LIS
__global__ __launch_bounds__(1024) void grid_scan_kernel(const int32_t* __restrict__ counts, int N,
                                                         int T, int K,
                                                         int32_t* __restrict__ offsets,
                                                         double* __restrict__ lis) {
  __shared__ int part[1024];
  __shared__ int mx[1024];
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int n0 = min(tid * per, N), n1 = min(n0 + per, N);
  int sum = 0, best = 0;
  for (int n = n0; n < n1; ++n) {
    sum += counts[n];
    best = max(best, counts[n]);
  }
  part[tid] = sum;
  mx[tid] = best;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan of segment sums
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
  for (int n = n0; n < n1; ++n) {
    offsets[n] = run;
    run += counts[n];
  }
  if (tid == 1023) offsets[N] = part[1023];
  if (tid == 0) *lis = T == 0 ? NAN : (double)((int64_t)N * mx[0]) / (double)((int64_t)T * K);
}

__global__ __launch_bounds__(256) void grid_write_kernel(const uint32_t* __restrict__ bits,
                                                         const int32_t* __restrict__ bitpre, int T,
                                                         int W, int K,
                                                         const int32_t* __restrict__ ccount,
                                                         const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ row_assign,
                                                         int32_t* __restrict__ assign_row) {
  const int wc = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  if (wc >= W) return;
  const int N = W * 32;
  int base[32];
#pragma unroll
  for (int q = 0; q < 32; ++q)
    base[q] = offsets[wc * 32 + q] + ccount[(size_t)c * N + wc * 32 + q];
  const int t1 = min((c + 1) * kPermChunkT, T);
  for (int t = c * kPermChunkT; t < t1; ++t) {
    const uint32_t w = bits[(size_t)t * W + wc];
    if (!w) continue;
    const int pre = bitpre[(size_t)t * W + wc];
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      if ((w >> q) & 1u) {
        const int row = base[q]++;
        const int a = t * K + pre + __popc(w & ((1u << q) - 1u));
        if (row_assign) row_assign[row] = a;
        if (assign_row) assign_row[a] = row;
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

hipError_t launch_log_softmax_rows(const float* l, int T, int n, float* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(log_softmax_kernel, dim3(T), dim3(64), 0, s, l, n, out);
  return hipGetLastError();
}

hipError_t launch_grid_topk(const float* pr, const float* pc, int T, int nr, int nc, int K,
                            int32_t* idx, float* gate, uint32_t* bits, int32_t* bitpre,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (nr > kGridMax || nc > kGridMax || nc % 32 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(grid_topk_kernel, dim3(T), dim3(256), 0, s, pr, pc, nr, nc, K, idx, gate,
                     bits, bitpre);
  return hipGetLastError();
}

size_t grid_permute_ws_bytes(int T, int N) {
  const size_t nchunk = (size_t)(T + kPermChunkT - 1) / kPermChunkT;
  return nchunk * (size_t)N * sizeof(int32_t);
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
  hipLaunchKernelGGL(grid_scan_kernel, dim3(1), dim3(1024), 0, s, counts, N, T, K, offsets, lis);
  if (T > 0) {
    const dim3 grid((unsigned)((W + 255) / 256), (unsigned)nchunk);
    hipLaunchKernelGGL(grid_write_kernel, grid, dim3(256), 0, s, bits, bitpre, T, W, K, ccount,
                       offsets, row_assign, assign_row);
  }
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* out, int n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(iota_kernel, dim3((n + 255) / 256), dim3(256), 0, s, out, n);
  return hipGetLastError();
}

}  // namespace moe
