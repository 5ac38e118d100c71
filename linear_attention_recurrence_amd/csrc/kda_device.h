// kda_device.h -- small device helpers shared by the libkda kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int D = 128;  // key and value head dimension

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): a 16-bit-significand pair
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo16, uint16_t hi16) {
  return (uint32_t)lo16 | ((uint32_t)hi16 << 16);
}

// 16x16x32 bf16 MFMA, fp32 accumulate. Lane l holds A[l%16][8*(l/16)+i] and
// B[8*(l/16)+i][l%16] (i < 8); the result D[4*(l/16)+r][l%16] (r < 4).
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint2 a, uint2 b) {
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

}  // namespace kda
