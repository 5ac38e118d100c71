// kda_probe.hip -- measurement probes, not part of the method. They give the rates the chip
// actually reaches on the simplest possible work, measured in the same run as the kernels they
// are compared with: a streaming copy and a streaming read (HBM bandwidth) and a loop of
// independent bf16 MFMAs (matrix-core rate).
//
// Copy and read: grid-stride over float4s, four non-temporal loads in flight per thread (the copy's
// stores non-temporal too: each byte is touched once). The read adds what each thread loaded and
// stores one float per thread, so that the loads have a use. A sweep of these shapes (1-8 loads in
// flight, 8-64 workgroups per CU, plain or non-temporal) found non-temporal access the only factor
// worth more than a few percent. MFMA: each wave keeps
// eight independent 16x16 accumulators and issues v_mfma_f32_16x16x32_bf16 on them in turn, so the
// matrix pipeline never waits on a result; each thread stores the sum of its accumulators.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) probe_copy_kernel(const f32x4v* __restrict__ s, f32x4v* __restrict__ d,
                                                         int64_t n) {
  const int64_t step = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * step < n; i += 4 * step) {
    f32x4v v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(s + i + u * step);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], d + i + u * step);
  }
  for (; i < n; i += step) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

__global__ void __launch_bounds__(256) probe_read_kernel(const f32x4v* __restrict__ s, int64_t n,
                                                         float* __restrict__ sink) {
  const int64_t step = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (; i + 3 * step < n; i += 4 * step) {
    f32x4v v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(s + i + u * step);
    a0 += v[0].x + v[0].y + v[0].z + v[0].w;
    a1 += v[1].x + v[1].y + v[1].z + v[1].w;
    a2 += v[2].x + v[2].y + v[2].z + v[2].w;
    a3 += v[3].x + v[3].y + v[3].z + v[3].w;
  }
  for (; i < n; i += step) {
    const f32x4v v = __builtin_nontemporal_load(s + i);
    a0 += v.x + v.y + v.z + v.w;
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = (a0 + a1) + (a2 + a3);
}

constexpr int kProbeBlock = 32;

__global__ void __launch_bounds__(256) probe_mfma_kernel(int iters, float seed, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(seed * (float)(lane + j));
    b[j] = (__bf16)(seed * (float)(lane - j));
  }
  // rounds in blocks of kProbeBlock, each block fully unrolled: the register allocator moves the
  // loop-carried accumulators at the loop edge, so the moves come once per block instead of per round
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; it += kProbeBlock) {
#pragma unroll
    for (int r = 0; r < kProbeBlock; ++r)
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = mfma16(a, b, acc[u]);
  }
  float t = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) t += (acc[u][0] + acc[u][1]) + (acc[u][2] + acc[u][3]);
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = t;
}

}  // namespace

hipError_t launch_probe_copy(const void* src, void* dst, int64_t n_f4, int grid, hipStream_t stream) {
  if (n_f4 <= 0) return hipSuccess;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const f32x4v*>(src),
                     static_cast<f32x4v*>(dst), n_f4);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, int64_t n_f4, float* sink, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const f32x4v*>(src), n_f4,
                     sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int iters, int grid, float seed, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(256), 0, stream, iters, seed, sink);
  return hipGetLastError();
}

}  // namespace kda
