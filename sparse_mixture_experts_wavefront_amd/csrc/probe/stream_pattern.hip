// stream_pattern.hip -- measurement probe (not part of libmoe): HBM read rate of
// the weight-read patterns of the decode kernels on MI355X.
//
// 470 MB of 2048-byte rows (the INT4 gate/up weights of the Mixtral decode
// workload).  "pat L D RW": blocks of 4 waves, each wave RW blocks of 16 rows
// (a block owns 64*RW rows); lane (r, g) of a load reads 16 bytes of row r at
// offset g*16 + j*64 of the current visit (the MFMA operand layout); one visit
// reads L*64 contiguous bytes of each row (L loads per row block issued
// together), D visits in flight.  "lin D": each wave instruction reads 1 KB
// contiguous, 256 rows per block.  Before every timed launch a 512 MB buffer is
// read, so the rows come from HBM.
//
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       sparse_mixture_experts_wavefront_amd/csrc/probe/stream_pattern.hip -o stream_pattern
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int L, int D, int RW = 4>
__global__ __launch_bounds__(256) void pat_kernel(const unsigned char* W, int row_bytes, uint32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const size_t strip = (size_t)blockIdx.x * 64 * RW * row_bytes;
  const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + strip), (short)0, 64 * RW * row_bytes, 0x00020000);
  uint32_t off[RW];
  for (int rb = 0; rb < RW; ++rb) off[rb] = (uint32_t)((w * 16 * RW + rb * 16 + r16) * row_bytes + g * 16);
  const int visits = row_bytes / (64 * L);
  u32x4 acc = {0, 0, 0, 0};
  u32x4 st[D][RW][L];
  auto load = [&](int d, int v) {
    const uint32_t vo = v < visits ? (uint32_t)v * 64 * L : 64u * RW * row_bytes;
#pragma unroll
    for (int rb = 0; rb < RW; ++rb)
#pragma unroll
      for (int j = 0; j < L; ++j)
        st[d][rb][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(res, (int)(off[rb] + vo + j * 64), 0, 0));
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);
  for (int v0 = 0; v0 < visits; v0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
#pragma unroll
      for (int rb = 0; rb < RW; ++rb)
#pragma unroll
        for (int j = 0; j < L; ++j) acc ^= st[u][rb][j];
      load(u, v0 + u + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  out[blockIdx.x * 256 + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// linear: each wave instruction reads 1 KB contiguous; same bytes per block
template <int D>
__global__ __launch_bounds__(256) void lin_kernel(const unsigned char* W, int row_bytes, uint32_t* out) {
  const int tid = threadIdx.x;
  const size_t strip = (size_t)blockIdx.x * 256 * row_bytes;
  const int bytes = 256 * row_bytes;
  const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + strip), (short)0, bytes, 0x00020000);
  const int steps = bytes / (256 * 16 * 4);  // 4 loads of 4 KB per block step
  u32x4 acc = {0, 0, 0, 0};
  u32x4 st[D][4];
  auto load = [&](int d, int v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t o = v < steps ? (uint32_t)(v * 4 + j) * 4096 + tid * 16 : (uint32_t)bytes;
      st[d][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(res, (int)o, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);
  for (int v0 = 0; v0 < steps; v0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= st[u][j];
      load(u, v0 + u + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  out[blockIdx.x * 256 + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("err %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)

int main() {
  const int row_bytes = 2048, rows = 229376, blocks = rows / 256;
  const size_t bytes = (size_t)rows * row_bytes;
  unsigned char* W; uint32_t* out; unsigned char* flush;
  const size_t fbytes = 512u << 20;
  CHECK(hipMalloc(&W, bytes));
  CHECK(hipMalloc(&out, (size_t)(rows / 64) * 256 * 4));
  CHECK(hipMalloc(&flush, fbytes));
  CHECK(hipMemset(W, 1, bytes));
  CHECK(hipMemset(flush, 2, fbytes));
  uint32_t* fo; CHECK(hipMalloc(&fo, (size_t)(fbytes / row_bytes / 256) * 256 * 4));
  hipEvent_t a, b; CHECK(hipEventCreate(&a)); CHECK(hipEventCreate(&b));
  auto run = [&](const char* name, auto kern, int reps, int nblocks = 0) -> int {
    const int gb = nblocks ? nblocks : blocks;
    float best = 1e9, sum = 0;
    for (int i = 0; i < reps + 1; ++i) {
      // read-flush the MALL with the linear kernel over the 512 MB buffer
      hipLaunchKernelGGL((lin_kernel<2>), dim3(fbytes / row_bytes / 256), dim3(256), 0, 0, flush, row_bytes, fo);
      CHECK(hipEventRecord(a, 0));
      hipLaunchKernelGGL(kern, dim3(gb), dim3(256), 0, 0, W, row_bytes, out);
      CHECK(hipEventRecord(b, 0));
      CHECK(hipEventSynchronize(b));
      float ms; CHECK(hipEventElapsedTime(&ms, a, b));
      if (i > 0) { best = ms < best ? ms : best; sum += ms; }
    }
    printf("%-16s best %.1f us  mean %.1f us  %.2f TB/s (best)\n", name, best * 1e3, sum / reps * 1e3, bytes / (best * 1e-3) / 1e12);
    fflush(stdout);
    return 0;
  };
  run("lin D2", lin_kernel<2>, 5);
  run("pat L1 D4 RW4", pat_kernel<1, 4, 4>, 5);
  run("pat L4 D2 RW4", pat_kernel<4, 2, 4>, 5);
  run("pat L1 D4 RW1", pat_kernel<1, 4, 1>, 5, rows / 64);
  run("pat L1 D8 RW1", pat_kernel<1, 8, 1>, 5, rows / 64);
  run("pat L4 D2 RW1", pat_kernel<4, 2, 1>, 5, rows / 64);
  run("pat L4 D4 RW1", pat_kernel<4, 4, 1>, 5, rows / 64);
  run("pat L1 D4 RW2", pat_kernel<1, 4, 2>, 5, rows / 128);
  run("pat L4 D2 RW2", pat_kernel<4, 2, 2>, 5, rows / 128);
  return 0;
}
