// kda_norm.hip -- the output gated RMSNorm on its own (for o written by kda_verify or
// kda_chunk_prefill); the arithmetic and its order are in kda_norm.h.
//
// One row = one (token, head), 128 fp32 values. A wave takes 4 rows; lane 16 r + s of a wave holds
// slice s of row r (two 16-byte loads of o, two 8-byte loads of the gate), so the loads cover
// 64-byte runs of each row. The 16 slice sums of a row are gathered into every lane of the row in
// slice order and added one by one.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_norm.h"

namespace kda {

namespace {

__global__ void __launch_bounds__(256) gated_rmsnorm_kernel(int64_t rows, const float* __restrict__ o,
                                                          const uint16_t* __restrict__ gate,
                                                          const float* __restrict__ w, float eps,
                                                          uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int s = lane & 15, wq = s >> 2, q = s & 3;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool ok = row < rows;
  const int64_t r = ok ? row : rows - 1;  // a lane past the end reads the last row and stores nothing
  const int ca = 32 * wq + 4 * q, cb = ca + 16;
  const float* orow = o + r * D;
  const uint16_t* grow = gate + r * D;
  const f32x4 a = *reinterpret_cast<const f32x4*>(orow + ca);
  const f32x4 b = *reinterpret_cast<const f32x4*>(orow + cb);
  const uint2 ga = *reinterpret_cast<const uint2*>(grow + ca);
  const uint2 gb = *reinterpret_cast<const uint2*>(grow + cb);
  const float4 wa = *reinterpret_cast<const float4*>(w + ca);
  const float4 wb = *reinterpret_cast<const float4*>(w + cb);
  const float part = norm_slice_ssq(a, b);
  float ss = 0.f;
  const int base = lane & ~15;
#pragma unroll
  for (int k = 0; k < 16; ++k) ss = ss + __shfl(part, base + k);
  const float rstd = norm_rstd(ss, eps);
  const uint2 ya = norm_apply4(a, ga, wa, rstd);
  const uint2 yb = norm_apply4(b, gb, wb, rstd);
  if (ok) {
    *reinterpret_cast<uint2*>(y + r * D + ca) = ya;
    *reinterpret_cast<uint2*>(y + r * D + cb) = yb;
  }
}

}  // namespace

hipError_t launch_gated_rmsnorm(int64_t rows, const float* o, const uint16_t* gate, const float* w, float eps,
                                uint16_t* y, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = (rows + 15) / 16;  // 16 rows per 256-thread block
  hipLaunchKernelGGL(gated_rmsnorm_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, rows, o, gate, w, eps, y);
  return hipGetLastError();
}

}  // namespace kda
