// kda_norm.h -- the arithmetic of the output gated RMSNorm, shared by the standalone kernel
// (kda_norm.hip) and the epilogue fused into the chunked prefill, so that both give the same bits.
//
// Source: Kimi K3 B200 deployment notes (zdszero.github.io), the prefill / decode kernel-fusion
// items: the KDA output goes through a gated RMSNorm that reads the attention output at its native
// stride, the one fusion there allowed fast math (tolerance 8e-3). The notes name the operation,
// not its formula; the plain reading used here is
//   y[j] = o[j] / sqrt(mean_j' o[j']^2 + eps) * w[j] * sigmoid(g[j]),   sigmoid(x) = 1 / (1 + e^-x),
// with w one weight per channel shared by all heads, and y rounded to bf16 (nearest even).
//
// Summation order (fixed, so both kernels agree bit for bit): a row of 128 values is cut into 16
// slices of 8, slice s = 4 w + q holding columns 32w + 4q + {0..3} and then 32w + 16 + 4q + {0..3};
// each slice's squares are summed in that order, then the 16 slice sums in the order of s.
#pragma once

#include "kda_device.h"

namespace kda {

// sum of squares of one slice: a = columns 32w + 4q + {0..3}, b = columns 32w + 16 + 4q + {0..3}
__device__ __forceinline__ float norm_slice_ssq(const f32x4& a, const f32x4& b) {
  float s = a[0] * a[0];
  s = s + a[1] * a[1];
  s = s + a[2] * a[2];
  s = s + a[3] * a[3];
  s = s + b[0] * b[0];
  s = s + b[1] * b[1];
  s = s + b[2] * b[2];
  s = s + b[3] * b[3];
  return s;
}

// 1 / sqrt(mean square + eps) from the row's sum of squares (hardware reciprocal square root)
__device__ __forceinline__ float norm_rstd(float ss, float eps) {
  return __builtin_amdgcn_rsqf(ss * (1.0f / 128.0f) + eps);
}

// sigmoid of a bf16 gate value (hardware exp2 and reciprocal)
__device__ __forceinline__ float norm_gate(uint32_t g_bf16) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(bf2f(g_bf16) * -1.4426950408889634f));
}

// four outputs of a row from o[c..c+3], the gate bits of the same columns (two packed pairs),
// w[c..c+3] and the row's 1/rms, as two packed bf16 pairs
__device__ __forceinline__ uint2 norm_apply4(const f32x4& o, uint2 gate, const float4& w, float rstd) {
  const float y0 = o[0] * rstd * w.x * norm_gate(gate.x & 0xffffu);
  const float y1 = o[1] * rstd * w.y * norm_gate(gate.x >> 16);
  const float y2 = o[2] * rstd * w.z * norm_gate(gate.y & 0xffffu);
  const float y3 = o[3] * rstd * w.w * norm_gate(gate.y >> 16);
  return make_uint2(pack2(f2bf(y0), f2bf(y1)), pack2(f2bf(y2), f2bf(y3)));
}

}  // namespace kda
