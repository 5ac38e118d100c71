// kda_step.h -- the token-by-token step of the KDA recurrence on a 256-thread
// workgroup, shared by every kernel whose results must agree bit for bit (the
// recurrent verify and its commit, the fold, the fused fold-then-verify).
//
// Sources: "SGLang and Miles Add Day-0 Support for Kimi K3" (LMSYS blog),
// section "ReplaySSM: raw-input replay for the KDA state" -- the fold is a
// verbatim clone of the verify recurrence (same tiles, same reduction order)
// on the stored gate values, bit-identical to the recurrent commit.
//
// Ownership: wave w, lane l holds rows 16*(l&7) .. +15 and columns
// 32*w + 4*(l>>3) .. +3 of the fp32 state S[128][128] (64 floats). Sums over
// the key channel are a sequential FMA chain over the thread's 16 rows, then a
// butterfly over the eight lanes l&7 that share the columns. Every product and
// sum is an explicit fmaf / mul / add (the files are built with
// -ffp-contract=off) and the decay is expf of the stored fp32 gk.
#pragma once

#include "kda_device.h"

namespace kda {

constexpr int TB = 8;  // steps staged in LDS per batch

struct alignas(16) StepLds {
  float a[TB][D];     // exp(gk)
  float ak[TB][D];    // exp(gk) * k
  float k[TB][D];
  float q[TB][D];     // verify only
  float v[TB][D];
  float beta[TB];
};

// the same staging without q, for folds
struct alignas(16) FoldLds {
  float a[TB][D];
  float ak[TB][D];
  float k[TB][D];
  float v[TB][D];
  float beta[TB];
};

// Stage one ring entry (bf16 k and v, fp32 gk and beta) of step tt for channels c4 .. c4+3, as
// every fold does: a = expf(gk), ak = a * k.
template <class SL>
__device__ __forceinline__ void stage_entry(SL& L, int tt, int c4, const uint2& kr, const uint2& vr, const float4& g4,
                                            float beta) {
  const float4 k4 = make_float4(bf2f(kr.x & 0xffffu), bf2f(kr.x >> 16), bf2f(kr.y & 0xffffu), bf2f(kr.y >> 16));
  const float4 v4 = make_float4(bf2f(vr.x & 0xffffu), bf2f(vr.x >> 16), bf2f(vr.y & 0xffffu), bf2f(vr.y >> 16));
  const float a0 = expf(g4.x), a1 = expf(g4.y), a2 = expf(g4.z), a3 = expf(g4.w);
  *reinterpret_cast<float4*>(&L.a[tt][c4]) = make_float4(a0, a1, a2, a3);
  *reinterpret_cast<float4*>(&L.ak[tt][c4]) = make_float4(a0 * k4.x, a1 * k4.y, a2 * k4.z, a3 * k4.w);
  *reinterpret_cast<float4*>(&L.k[tt][c4]) = k4;
  *reinterpret_cast<float4*>(&L.v[tt][c4]) = v4;
  if (c4 == 0) L.beta[tt] = beta;
}

#define KDA_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), (ctrl), 0xf, 0xf, false))

// sum over the 8 lanes (l & 7) of a row group; every lane gets the same bits
__device__ __forceinline__ float red8(float x) {
  x = x + KDA_DPP(x, 0xB1);   // quad_perm [1,0,3,2]
  x = x + KDA_DPP(x, 0x4E);   // quad_perm [2,3,0,1]
  x = x + KDA_DPP(x, 0x141);  // row_half_mirror: the other quad of the 8
  return x;
}

// One recurrence step on this thread's 16x4 block of S (decay, delta update).
// u_j = sum_c a_c k_c S_cj ; w_j = beta (v_j - u_j) ; S_cj = a_c S_cj + k_c w_j
// SL: any LDS block with the members a, ak, k, v [.][D] and beta[.] of StepLds
template <class SL>
__device__ __forceinline__ void step_update(float (&S)[16][4], const SL& L, int tt, int r0, int col0) {
  float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 ak = *reinterpret_cast<const float4*>(&L.ak[tt][r0 + 4 * i4]);
    const float akv[4] = {ak.x, ak.y, ak.z, ak.w};
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = __builtin_fmaf(akv[ii], S[4 * i4 + ii][j], u[j]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = red8(u[j]);
  const float4 v4 = *reinterpret_cast<const float4*>(&L.v[tt][col0]);
  const float beta = L.beta[tt];
  float w[4];
  w[0] = beta * (v4.x - u[0]);
  w[1] = beta * (v4.y - u[1]);
  w[2] = beta * (v4.z - u[2]);
  w[3] = beta * (v4.w - u[3]);
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 a4 = *reinterpret_cast<const float4*>(&L.a[tt][r0 + 4 * i4]);
    const float4 k4 = *reinterpret_cast<const float4*>(&L.k[tt][r0 + 4 * i4]);
    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
    const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[4 * i4 + ii][j] = __builtin_fmaf(av[ii], S[4 * i4 + ii][j], kv[ii] * w[j]);
  }
}

__device__ __forceinline__ void load_state(float (&S)[16][4], const float* __restrict__ src, int r0, int col0) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 x = *reinterpret_cast<const float4*>(src + (size_t)(r0 + i) * D + col0);
    S[i][0] = x.x; S[i][1] = x.y; S[i][2] = x.z; S[i][3] = x.w;
  }
}

__device__ __forceinline__ void store_state(const float (&S)[16][4], float* __restrict__ dst, int r0, int col0) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    *reinterpret_cast<float4*>(dst + (size_t)(r0 + i) * D + col0) = make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
}

}  // namespace kda
