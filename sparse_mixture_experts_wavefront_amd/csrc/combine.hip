// combine.hip -- weighted combine back to token order.
//
// The grouped FFN leaves one gate-scaled output row per (token, slot) in
// expert-major order; the combine gathers a token's k rows through assign_row
// and sums them in slot order j = 0..k-1, then adds the always-active shared
// experts ("OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale"
// -- abstract and Figure 1: a shared dense branch next to the routed one).  The
// fixed order makes the result bitwise reproducible.
//
// HBM-bound: each output float reads k rows (+1 shared) and writes once.  One
// 64-lane block per (token, 256 columns), 4 floats (16 bytes) per lane per
// access, so a decode step of a few tokens still spreads over many CUs.  When
// the down pass split its reduction, each row arrives as nsplit partial rows and
// the combine adds them too (slot-major, slice-minor order); the partial rows of
// one slot are loaded four at a time and added in that order.  Rows may be bf16
// (MOE_F_BF16_ROWS): widened to fp32 exactly before the same sum.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCombCols = 256;  // columns per block (64 lanes x 4)
constexpr int kCombSplitMin = 8;  // K slices per row from which four waves share a row's slices

__device__ __forceinline__ void add4(float4& s, const float4 v) {
  s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
}

// four values of a row: fp32, or bf16 rows (MOE_F_BF16_ROWS) widened exactly
template <bool BF16ROWS>
__device__ __forceinline__ float4 load_row4(const float* rows, size_t idx) {
  if constexpr (BF16ROWS) {
    const uint2 v = *(const uint2*)((const u16*)rows + idx);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
  } else {
    return *(const float4*)(rows + idx);
  }
}

// y[t][i..i+3]: the k rows of token t (each as nsplit partial rows), then the
// shared term, added in that fixed order
template <bool BF16OUT, bool BF16ROWS>
__device__ __forceinline__ void combine_one(const float* __restrict__ y_rows,
                                            const int32_t* __restrict__ assign_row, int k, int d,
                                            const float* __restrict__ y_shared, void* yv,
                                            int nsplit, size_t split_stride, size_t t, int i) {
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  bool first = true;
  auto add = [&](const float4 v) {
    if (first) {
      s = v;
      first = false;
    } else {
      add4(s, v);
    }
  };
  for (int j = 0; j < k; ++j) {
    const size_t base = (size_t)assign_row[t * k + j] * d + i;
    int sp = 0;
    for (; sp + 4 <= nsplit; sp += 4) {
      float4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = load_row4<BF16ROWS>(y_rows, base + (size_t)(sp + q) * split_stride);
#pragma unroll
      for (int q = 0; q < 4; ++q) add(v[q]);
    }
    for (; sp < nsplit; ++sp) add(load_row4<BF16ROWS>(y_rows, base + (size_t)sp * split_stride));
  }
  if (y_shared) add4(s, *(const float4*)(y_shared + t * d + i));
  if constexpr (BF16OUT) {
    u16* y = (u16*)yv + t * d + i;
    const uint32_t lo = (uint32_t)f32_to_bf16(s.x) | ((uint32_t)f32_to_bf16(s.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(s.z) | ((uint32_t)f32_to_bf16(s.w) << 16);
    *(uint2*)y = make_uint2(lo, hi);
  } else {
    *(float4*)((float*)yv + t * d + i) = s;
  }
}

// work item b = (token b / nchunk, columns of chunk b % nchunk); grid-stride
template <bool BF16OUT, bool BF16ROWS>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ y_rows,
                                                     const int32_t* __restrict__ assign_row,
                                                     int k, int d,
                                                     const float* __restrict__ y_shared,
                                                     void* __restrict__ yv, int nsplit,
                                                     size_t split_stride, size_t work_items) {
  const int nchunk = (d + kCombCols - 1) / kCombCols;
  for (size_t b = blockIdx.x; b < work_items; b += gridDim.x) {
    const size_t t = b / nchunk;
    const int i = (int)(b - t * nchunk) * kCombCols + threadIdx.x * 4;
    if (i < d)
      combine_one<BF16OUT, BF16ROWS>(y_rows, assign_row, k, d, y_shared, yv, nsplit, split_stride,
                                     t, i);
  }
}

// Many K slices per row (the sparse down-projection writes up to 32): the four
// waves of a block take a quarter of each row's slices each (every slot in
// order, its slices in order), then wave 0 adds the four partial sums in wave
// order and the shared term -- a fixed order, so the result is deterministic,
// with a quarter of the dependent loads per lane.
template <bool BF16OUT, bool BF16ROWS>
__global__ __launch_bounds__(256) void combine_split_kernel(const float* __restrict__ y_rows,
                                                            const int32_t* __restrict__ assign_row,
                                                            int k, int d,
                                                            const float* __restrict__ y_shared,
                                                            void* __restrict__ yv, int nsplit,
                                                            size_t split_stride, size_t work_items) {
  __shared__ float4 part[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nchunk = (d + kCombCols - 1) / kCombCols;
  const int s0 = w * nsplit / 4, s1 = (w + 1) * nsplit / 4;
  for (size_t b = blockIdx.x; b < work_items; b += gridDim.x) {
    const size_t t = b / nchunk;
    const int i = (int)(b - t * nchunk) * kCombCols + lane * 4;
    const bool ok = i < d;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ok) {
      for (int j = 0; j < k; ++j) {
        const size_t base = (size_t)assign_row[t * k + j] * d + i;
        int sp = s0;
        for (; sp + 4 <= s1; sp += 4) {
          float4 v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = load_row4<BF16ROWS>(y_rows, base + (size_t)(sp + q) * split_stride);
#pragma unroll
          for (int q = 0; q < 4; ++q) add4(s, v[q]);
        }
        for (; sp < s1; ++sp) add4(s, load_row4<BF16ROWS>(y_rows, base + (size_t)sp * split_stride));
      }
    }
    part[w][lane] = s;
    __syncthreads();
    if (w == 0 && ok) {
      float4 y = part[0][lane];
      add4(y, part[1][lane]);
      add4(y, part[2][lane]);
      add4(y, part[3][lane]);
      if (y_shared) add4(y, *(const float4*)(y_shared + t * d + i));
      if constexpr (BF16OUT) {
        u16* o = (u16*)yv + t * d + i;
        const uint32_t lo = (uint32_t)f32_to_bf16(y.x) | ((uint32_t)f32_to_bf16(y.y) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(y.z) | ((uint32_t)f32_to_bf16(y.w) << 16);
        *(uint2*)o = make_uint2(lo, hi);
      } else {
        *(float4*)((float*)yv + t * d + i) = y;
      }
    }
    __syncthreads();  // part is rewritten by the next item
  }
}

}  // namespace

hipError_t launch_combine(const float* y_rows, const int32_t* assign_row, int T, int k, int d,
                          const float* y_shared, void* y, moe_dtype ydt, hipStream_t s,
                          int nsplit, size_t split_stride, bool rows_bf16) {
  if (T == 0) return hipSuccess;
  // one block per (token, 256 columns), at most 2^20 blocks (grid-stride beyond)
  const size_t items = (size_t)((d + kCombCols - 1) / kCombCols) * (size_t)T;
  const dim3 grid((unsigned)(items < (1u << 20) ? items : (1u << 20)));
#define MOE_COMBINE(O, R)                                                                    \
  hipLaunchKernelGGL((combine_kernel<O, R>), grid, dim3(64), 0, s, y_rows, assign_row, k, d, \
                     y_shared, y, nsplit, split_stride, items)
#define MOE_COMBINE_SPLIT(O, R)                                                          \
  hipLaunchKernelGGL((combine_split_kernel<O, R>), grid, dim3(256), 0, s, y_rows, assign_row, \
                     k, d, y_shared, y, nsplit, split_stride, items)
  if (nsplit >= kCombSplitMin) {
    if (ydt == MOE_DT_BF16) {
      if (rows_bf16) MOE_COMBINE_SPLIT(true, true); else MOE_COMBINE_SPLIT(true, false);
    } else {
      if (rows_bf16) MOE_COMBINE_SPLIT(false, true); else MOE_COMBINE_SPLIT(false, false);
    }
  } else if (ydt == MOE_DT_BF16) {
    if (rows_bf16) MOE_COMBINE(true, true); else MOE_COMBINE(true, false);
  } else {
    if (rows_bf16) MOE_COMBINE(false, true); else MOE_COMBINE(false, false);
  }
#undef MOE_COMBINE_SPLIT
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
