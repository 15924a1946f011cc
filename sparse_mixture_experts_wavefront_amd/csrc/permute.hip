// permute.hip -- expert-centric permutation, per-expert counts and the Load
// Imbalance Score.
//
// "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale" -- What
// carries the argument and Figure 3: execution is inverted from token order to
// expert order, active experts are compressed into contiguous groups so that
// each group runs as one dense GEMM.
// "A Replicate-and-Quantize Strategy for Plug-and-Play Load Balancing of Sparse
// Mixture-of-Experts LLMs" -- Definition 1 (quoted in its Circularity Check):
// n_j = tokens routed to expert j, LIS = m * max_j n_j / (n * k).
//
// Flat assignment a = t*k + j carries expert topk_idx[a].  Rows are grouped by
// expert; inside a group they keep ascending a (a stable counting sort).
//   histogram : per-block expert counts with LDS integer atomics (order-free)
//   scan      : one wave scans blocks then experts -> offsets, block bases, LIS
//   scatter   : each block walks its chunk in rounds of 256 in a order; a
//               lane's rank among equal experts in its wave comes from a
//               match-any built out of log2(64) ballots, earlier waves of the
//               round add their per-expert counts from LDS.
// Assignments of at most kPermFusedMax entries take one fused block (decode
// latency); up to kPermFusedBigMax one 1024-thread block that ranks every
// 64-assignment chunk at once (prefill latency); larger ones the three-kernel
// path.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

__device__ __forceinline__ unsigned long long lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? ((~0ull) >> (64 - lane)) : 0ull;
}

// Lanes of this wave holding the same valid expert id as this lane.
__device__ __forceinline__ unsigned long long match_expert(int e, bool valid) {
  unsigned long long m = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 6; ++bit) {
    const bool b = (e >> bit) & 1;
    const unsigned long long bal = __ballot(valid && b);
    m &= b ? bal : ~bal;
  }
  return m;
}

__device__ void write_lis(double* lis, int T, int E, int k, int maxc) {
  if (lis) *lis = (T == 0) ? (double)NAN : (double)((long long)E * maxc) / (double)((long long)T * k);
}

// Scatter the assignments [begin, end) in rounds of 256, starting from the
// per-expert running row `run` (LDS).  All threads of the block call it.
__device__ void scatter_range(const int32_t* __restrict__ idx, int begin, int end, int E,
                              int* run, int (*wc)[kMaxExperts], int32_t* __restrict__ row_assign,
                              int32_t* __restrict__ assign_row) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  for (int r0 = begin; r0 < end; r0 += kBlock) {
    const int a = r0 + tid;
    int e = (a < end) ? idx[a] : -1;
    const bool valid = (e >= 0) && (e < E);
    if (!valid) e = 0;
    const unsigned long long m = match_expert(e, valid);
    const int rank = __popcll(m & lanemask_lt());
    const int cnt = __popcll(m);
    wc[w][lane] = 0;
    __syncthreads();
    if (valid && rank == 0) wc[w][e] = cnt;
    __syncthreads();
    if (valid) {
      int row = run[e] + rank;
      for (int ww = 0; ww < w; ++ww) row += wc[ww][e];
      if (row_assign) row_assign[row] = a;
      if (assign_row) assign_row[a] = row;
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) add += wc[ww][tid];
      run[tid] += add;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBlock) void permute_fused_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_assign,
    int32_t* __restrict__ assign_row, double* __restrict__ lis) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int run[kMaxExperts];
  __shared__ int wc[kWaves][kMaxExperts];
  const int tid = threadIdx.x, n = T * k;
  if (tid < kMaxExperts) cnt[tid] = 0;
  __syncthreads();
  for (int a = tid; a < n; a += kBlock) {
    const int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid < 64) {  // wave 0: exclusive scan and max over experts
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
      run[tid] = incl - c;
    }
    if (tid == E - 1) offsets[E] = incl;
    if (tid == 0) write_lis(lis, T, E, k, mx);
  }
  __syncthreads();
  scatter_range(idx, 0, n, E, run, wc, row_assign, assign_row);
}

// One 1024-thread block for kPermFusedMax < n <= kPermFusedBigMax.  Chunk c
// holds assignments [64c, 64c + 64) and belongs to wave c % 16.  (1) each wave
// ranks its chunks' lanes among equal experts (match-any from ballots) and the
// lane of rank 0 records the chunk's count of that expert; (2) per expert, an
// exclusive scan over chunks in chunk order (16 parts of consecutive chunks,
// lane = expert) turns the counts into each chunk's first row inside the
// expert; (3) wave 0 scans the expert totals into offsets, counts and LIS;
// (4) row = offsets[e] + chunk base + rank.  Rows inside an expert therefore
// follow the flat order a, as in the other paths.
constexpr int kBigBlock = 1024;
constexpr int kBigWaves = kBigBlock / 64;
constexpr int kBigChunks = kPermFusedBigMax / 64;
constexpr int kBigPer = kBigChunks / kBigWaves;  // chunks per wave
static_assert(kBigChunks % kBigWaves == 0 && kMaxExperts == 64,
              "chunks split evenly over the waves; one lane per expert");

__global__ __launch_bounds__(kBigBlock) void permute_fused_big_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_assign,
    int32_t* __restrict__ assign_row, double* __restrict__ lis) {
  __shared__ int cc[kBigChunks][kMaxExperts];  // chunk counts, then chunk bases
  __shared__ int part[kBigWaves][kMaxExperts];  // per-part sums
  __shared__ int off[kMaxExperts];              // expert totals, then offsets
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n = T * k, nch = (n + 63) >> 6;
  int ev[kBigPer];
#pragma unroll
  for (int j = 0; j < kBigPer; ++j) {
    const int a = (w + j * kBigWaves) * 64 + lane;
    ev[j] = a < n ? idx[a] : -1;
  }
  for (int i = tid; i < nch * kMaxExperts; i += kBigBlock) cc[i / kMaxExperts][i % kMaxExperts] = 0;
  __syncthreads();
  int rk[kBigPer];
#pragma unroll
  for (int j = 0; j < kBigPer; ++j) {
    const bool valid = ev[j] >= 0 && ev[j] < E;
    const int e = valid ? ev[j] : 0;
    const unsigned long long m = match_expert(e, valid);
    rk[j] = __popcll(m & lanemask_lt());
    if (valid && rk[j] == 0) cc[w + j * kBigWaves][e] = __popcll(m);
    if (!valid) ev[j] = -1;
  }
  __syncthreads();
  // part w = chunks [c0, c1); lane = expert
  const int S = (nch + kBigWaves - 1) / kBigWaves;
  const int c0 = min(nch, w * S), c1 = min(nch, c0 + S);
  int sum = 0;
  for (int c = c0; c < c1; ++c) sum += cc[c][lane];
  part[w][lane] = sum;
  __syncthreads();
  int base = 0;
  for (int q = 0; q < w; ++q) base += part[q][lane];
  for (int c = c0; c < c1; ++c) {
    const int v = cc[c][lane];
    cc[c][lane] = base;
    base += v;
  }
  if (w == kBigWaves - 1) off[lane] = base;  // the expert's total
  __syncthreads();
  if (w == 0) {
    const int c = (lane < E) ? off[lane] : 0;
    int incl = c;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int mx = c;
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
    off[lane] = incl - c;
    if (lane < E) {
      counts[lane] = c;
      offsets[lane] = incl - c;
    }
    if (lane == E - 1) offsets[E] = incl;
    if (lane == 0) write_lis(lis, T, E, k, mx);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBigPer; ++j) {
    if (ev[j] < 0) continue;
    const int c = w + j * kBigWaves, a = c * 64 + lane;
    const int row = off[ev[j]] + cc[c][ev[j]] + rk[j];
    if (row_assign) row_assign[row] = a;
    if (assign_row) assign_row[a] = row;
  }
}

__global__ __launch_bounds__(kBlock) void permute_hist_kernel(const int32_t* __restrict__ idx,
                                                              int n, int E,
                                                              int32_t* __restrict__ blk_counts) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x;
  if (tid < kMaxExperts) cnt[tid] = 0;
  __syncthreads();
  const int begin = blockIdx.x * kPermChunk, end = min(n, begin + kPermChunk);
  for (int a = begin + tid; a < end; a += kBlock) {
    const int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid < E) blk_counts[(size_t)blockIdx.x * E + tid] = cnt[tid];
}

__global__ __launch_bounds__(64) void permute_scan_kernel(const int32_t* __restrict__ blk_counts,
                                                          int nblk, int T, int E, int k,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ blk_base,
                                                          double* __restrict__ lis) {
  // lane e = expert: its per-block counts, 16 loads in flight per batch (the
  // counts come from the previous launch: a memory round trip per batch, not
  // per block).  Pass 1 totals them, pass 2 (after the scan over experts)
  // reads them again and writes each block's first row.
  constexpr int kBatch = 16;
  const int e = threadIdx.x;
  auto batch = [&](int b0, int (&v)[kBatch]) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      v[j] = (e < E && b0 + j < nblk) ? blk_counts[(size_t)(b0 + j) * E + e] : 0;
  };
  int c = 0;
  for (int b0 = 0; b0 < nblk; b0 += kBatch) {
    int v[kBatch];
    batch(b0, v);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) c += v[j];
  }
  int incl = c;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (e >= o) incl += v;
  }
  const int excl = incl - c;
  int mx = c;
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
  if (e < E) {
    counts[e] = c;
    offsets[e] = excl;
    int run = excl;
    for (int b0 = 0; b0 < nblk; b0 += kBatch) {
      int v[kBatch];
      batch(b0, v);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (b0 + j < nblk) blk_base[(size_t)(b0 + j) * E + e] = run;
        run += v[j];
      }
    }
  }
  if (e == E - 1) offsets[E] = incl;
  if (e == 0) write_lis(lis, T, E, k, mx);
}

__global__ __launch_bounds__(kBlock) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int n, int E, const int32_t* __restrict__ blk_base,
    int32_t* __restrict__ row_assign, int32_t* __restrict__ assign_row) {
  __shared__ int run[kMaxExperts];
  __shared__ int wc[kWaves][kMaxExperts];
  const int tid = threadIdx.x;
  if (tid < E) run[tid] = blk_base[(size_t)blockIdx.x * E + tid];
  __syncthreads();
  const int begin = blockIdx.x * kPermChunk, end = min(n, begin + kPermChunk);
  scatter_range(idx, begin, end, E, run, wc, row_assign, assign_row);
}

}  // namespace

size_t permute_ws_bytes(int T, int E, int k) {
  const long long n = (long long)T * k;
  if (n <= kPermFusedBigMax) return 0;
  const long long nblk = (n + kPermChunk - 1) / kPermChunk;
  return (size_t)(2 * nblk * E * sizeof(int32_t));
}

hipError_t launch_permute(const int32_t* idx, int T, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* row_assign, int32_t* assign_row,
                          double* lis, void* ws, hipStream_t s) {
  const int n = T * k;
  if (n <= kPermFusedMax) {
    hipLaunchKernelGGL(permute_fused_kernel, dim3(1), dim3(kBlock), 0, s, idx, T, E, k, counts,
                       offsets, row_assign, assign_row, lis);
    return hipGetLastError();
  }
  if (n <= kPermFusedBigMax) {
    hipLaunchKernelGGL(permute_fused_big_kernel, dim3(1), dim3(kBigBlock), 0, s, idx, T, E, k,
                       counts, offsets, row_assign, assign_row, lis);
    return hipGetLastError();
  }
  const int nblk = (n + kPermChunk - 1) / kPermChunk;
  int32_t* blk_counts = (int32_t*)ws;
  int32_t* blk_base = blk_counts + (size_t)nblk * E;
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nblk), dim3(kBlock), 0, s, idx, n, E, blk_counts);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(64), 0, s, blk_counts, nblk, T, E, k,
                     counts, offsets, blk_base, lis);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(kBlock), 0, s, idx, n, E, blk_base,
                     row_assign, assign_row);
  return hipGetLastError();
}

// ---- replica dispatch -------------------------------------------------------
// "A Replicate-and-Quantize Strategy for Plug-and-Play Load Balancing of Sparse
// Mixture-of-Experts LLMs" -- What carries the argument: a quantized copy of the
// heaviest-loaded expert is appended to the layer.  The pages leave the split of
// that expert's tokens open; here its assignments alternate in flat order
// a = t*k + j: even ranks stay, odd ranks go to the replica, slot E.  The
// expert-major layout over E+1 slots follows from the E-slot one without a new
// sort: the heavy expert keeps its even ranks in order at its start, experts
// after it move down by h = floor(n_heavy / 2) rows, and the odd ranks fill the
// last h rows (slot E) in order -- the stable expert-major order of the split
// routing, with counts, offsets and LIS (m = E + 1) to match.
__global__ __launch_bounds__(256) void replica_remap_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ assign_row, int n, int E,
    int heavy, int T, int k, int32_t* __restrict__ idx_out, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ row_assign_out,
    int32_t* __restrict__ assign_row_out, double* __restrict__ lis_out) {
  const int nh = counts[heavy], h = nh / 2;
  const int hstart = offsets[heavy];
  const int rep0 = n - h;  // first row of slot E
  if (blockIdx.x == 0) {
    // counts and offsets over E+1 slots, LIS with m = E + 1
    if (threadIdx.x <= E) {
      const int e = threadIdx.x;
      const int c = (e == E) ? h : (e == heavy ? nh - h : counts[e]);
      if (counts_out) counts_out[e] = c;
      if (offsets_out) offsets_out[e] = (e == E) ? rep0 : offsets[e] - (e > heavy ? h : 0);
    }
    if (threadIdx.x == 0) {
      if (offsets_out) offsets_out[E + 1] = n;
      int mx = h;
      for (int e = 0; e < E; ++e) mx = max(mx, e == heavy ? nh - h : counts[e]);
      if (lis_out)
        *lis_out = (T == 0) ? __builtin_nan("") : (double)((long long)(E + 1) * mx) / (double)((long long)T * k);
    }
  }
  for (int a = blockIdx.x * blockDim.x + threadIdx.x; a < n; a += gridDim.x * blockDim.x) {
    const int e = idx[a];
    const int row = assign_row[a];
    int e2 = e, row2;
    if (e == heavy) {
      const int rank = row - hstart;
      if (rank & 1) {
        e2 = E;
        row2 = rep0 + (rank >> 1);
      } else {
        row2 = hstart + (rank >> 1);
      }
    } else {
      row2 = row - (e > heavy ? h : 0);
    }
    if (idx_out) idx_out[a] = e2;
    if (assign_row_out) assign_row_out[a] = row2;
    if (row_assign_out) row_assign_out[row2] = a;
  }
}

hipError_t launch_replica_remap(const int32_t* idx, const int32_t* counts, const int32_t* offsets,
                                const int32_t* assign_row, int T, int E, int k, int heavy,
                                int32_t* idx_out, int32_t* counts_out, int32_t* offsets_out,
                                int32_t* row_assign_out, int32_t* assign_row_out, double* lis_out,
                                hipStream_t s) {
  const int n = T * k;
  const int blocks = max(1, min((n + 255) / 256, 1024));
  hipLaunchKernelGGL(replica_remap_kernel, dim3(blocks), dim3(256), 0, s, idx, counts, offsets,
                     assign_row, n, E, heavy, T, k, idx_out, counts_out, offsets_out,
                     row_assign_out, assign_row_out, lis_out);
  return hipGetLastError();
}

// ---- (expert, width) groups of nested low-bit experts ----------------------
// "D^2MoE: Dual Routing and Dynamic Scheduling for Efficient On-Device
// MoE-based LLM Serving" -- What carries the argument: each assignment carries a
// bit width, and the rows of one expert are run per width.  Group id
// 3*e + (width - 2); the permutation over the 3E ids then orders rows by expert,
// by width inside an expert, by flat assignment inside a group.
__global__ __launch_bounds__(256) void mwq_group_ids_kernel(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ widths,
                                                            int n, int32_t* __restrict__ out) {
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a < n) out[a] = 3 * idx[a] + min(max(widths[a], 2), 4) - 2;
}

hipError_t launch_mwq_group_ids(const int32_t* idx, const int32_t* widths, int n, int32_t* out,
                                hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mwq_group_ids_kernel, dim3((n + 255) / 256), dim3(256), 0, s, idx, widths, n,
                     out);
  return hipGetLastError();
}

}  // namespace moe
