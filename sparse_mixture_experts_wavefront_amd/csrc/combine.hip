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
// 256-thread block per token, 4 floats (16 bytes) per lane per access.  When the
// down GEMM split its reduction over K, each row arrives as nsplit partial rows
// and the combine adds them too (slot-major, slice-minor order).
#include "moe_internal.h"

namespace moe {
namespace {

template <bool BF16OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_rows,
                                                      const int32_t* __restrict__ assign_row,
                                                      int k, int d,
                                                      const float* __restrict__ y_shared,
                                                      void* __restrict__ yv, int nsplit,
                                                      size_t split_stride) {
  const int t = blockIdx.x;
  __shared__ int rows[kMaxTopK];
  if (threadIdx.x < k) rows[threadIdx.x] = assign_row[(size_t)t * k + threadIdx.x];
  __syncthreads();
  for (int i = threadIdx.x * 4; i < d; i += blockDim.x * 4) {
    float4 s = *(const float4*)(y_rows + (size_t)rows[0] * d + i);
    for (int sp = 1; sp < nsplit; ++sp) {
      const float4 v = *(const float4*)(y_rows + sp * split_stride + (size_t)rows[0] * d + i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    for (int j = 1; j < k; ++j) {
      for (int sp = 0; sp < nsplit; ++sp) {
        const float4 v = *(const float4*)(y_rows + sp * split_stride + (size_t)rows[j] * d + i);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
      }
    }
    if (y_shared) {
      const float4 v = *(const float4*)(y_shared + (size_t)t * d + i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    if constexpr (BF16OUT) {
      u16* y = (u16*)yv + (size_t)t * d + i;
      const uint32_t lo = (uint32_t)f32_to_bf16(s.x) | ((uint32_t)f32_to_bf16(s.y) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(s.z) | ((uint32_t)f32_to_bf16(s.w) << 16);
      *(uint2*)y = make_uint2(lo, hi);
    } else {
      *(float4*)((float*)yv + (size_t)t * d + i) = s;
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* y_rows, const int32_t* assign_row, int T, int k, int d,
                          const float* y_shared, void* y, moe_dtype ydt, hipStream_t s,
                          int nsplit, size_t split_stride) {
  if (T == 0) return hipSuccess;
  if (ydt == MOE_DT_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(256), 0, s, y_rows, assign_row, k, d,
                       y_shared, y, nsplit, split_stride);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(256), 0, s, y_rows, assign_row, k, d,
                       y_shared, y, nsplit, split_stride);
  return hipGetLastError();
}

}  // namespace moe
