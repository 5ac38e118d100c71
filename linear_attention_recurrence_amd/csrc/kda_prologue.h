// kda_prologue.h -- the per-element arithmetic of the KDA prologue (SiLU and sigmoid, the decay gate
// gk = -softplus, the per-head sum over a DPP row, bf16 conversions), shared by the prologue kernel and
// the fused decode kernel so that both give the same bits.
//
// Source: Kimi K3 B200 deployment notes (zdszero.github.io), the prefill / decode kernel-fusion items
// (the short conv with its SiLU and conv-state carry, beta's sigmoid). The gate formula is a reading:
// gk = -softplus(g), so exp(gk) = sigmoid(-g) is a decay in (0, 1).
#pragma once

#include "kda_device.h"

namespace kda {

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// two floats to a bf16 pair, nearest even (one v_cvt_pk_bf16_f32 on gfx950), the first in the low half
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}

// SiLU and the sigmoid through the hardware exp2 and reciprocal (the outputs are bf16, so their ~1 ulp
// errors vanish in the rounding); gk through an accurate form, since it feeds the recurrence's decay
__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}
// -softplus(g) = -(max(g, 0) + log(1 + x)) with x = e^-|g| in (0, 1]. log(1 + x) = 2 atanh(s) with
// s = x / (2 + x) in (0, 1/3], by the odd series 2 (s + s^3/3 + ... + s^11/11): the first omitted
// term is below 2 (1/3)^13 / 13 < 1e-7 of log 2, and every term is positive, so there is no
// cancellation for any x, the tiny ones included.
__device__ __forceinline__ float neg_softplus(float g) {
  const float x = __builtin_amdgcn_exp2f(fabsf(g) * -1.4426950408889634f);
  const float sv = x * __builtin_amdgcn_rcpf(2.0f + x);
  const float z = sv * sv;
  float poly = __builtin_fmaf(z, 2.0f / 11.0f, 2.0f / 9.0f);
  poly = __builtin_fmaf(z, poly, 2.0f / 7.0f);
  poly = __builtin_fmaf(z, poly, 2.0f / 5.0f);
  poly = __builtin_fmaf(z, poly, 2.0f / 3.0f);
  poly = __builtin_fmaf(z, poly, 2.0f);
  return -__builtin_fmaf(sv, poly, fmaxf(g, 0.0f));
}

// sum over the 16 lanes of a DPP row, as every lane's value (inclusive scan by row shifts, then lane 15
// of the row broadcast to it)
__device__ __forceinline__ float row_sum16(float v) {
  v = v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x111, 0xf, 0xf, true));
  v = v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x112, 0xf, 0xf, true));
  v = v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x114, 0xf, 0xf, true));
  v = v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x118, 0xf, 0xf, true));
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x15F, 0xf, 0xf, true));
}

// a row of 8 bf16 channels widened to fp32 (exact)
__device__ __forceinline__ void widen8(const uint4& r, float* f) {
  const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(wd[i] << 16);
    f[2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
  }
}

}  // namespace kda
