// kda_decode.hip -- one decode step of a KDA layer in one launch: the prologue of the new token (short
// conv with the conv state, SiLU, q/k L2 norm, beta and gk), the recurrent step with its readout and
// the commit written in place, and the output gated RMSNorm.
//
// Source: Kimi K3 B200 deployment notes (zdszero.github.io), the decode items of the optimisation
// timeline: a fused KDA decode kernel (conv + KDA + output norm in one launch) for the batch-1 shape,
// where the decode step is bound by launch latency. The readings are those of the separate kernels:
// the prologue's conv, SiLU, norms and gates, the recurrence of the verify kernel, and the gated
// RMSNorm of the norm kernel.
//
// Every part runs the arithmetic of the kernel it replaces, in the same order: the prologue's
// conv/SiLU/norm on 16 lanes per projection with the same DPP row sum, q/k/v rounded to bf16 as the
// prologue stores them; the verify kernel's staging (exp of gk, k widened from bf16) and step on the
// shared step function with the same lane ownership; the norm kernel's slice order. So y, the
// committed state and the conv state equal those of kda_prologue, kda_verify (n_tok = 1, commit in
// place) and kda_gated_rmsnorm run one after another, bit for bit.
//
// One 256-thread workgroup per (request, head). Wave 0: lanes 16 j + c (j = 0, 1, 2 for q, k, v) hold
// channels 8c .. 8c + 7 of projection j, while wave 1 computes exp(gk) and wave 3 fetches the output
// gate and norm weights, so that their loads overlap; wave 3 applies the norm at the end. A request whose
// slot is outside [0, n_slots) is skipped whole (its conv state is not touched).
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_norm.h"
#include "kda_prologue.h"
#include "kda_step.h"

namespace kda {

namespace {

// 16-byte aligned, and beta after o: o is read and written as 16-byte vectors
struct alignas(16) DecodeLds {
  float a[1][D];
  float ak[1][D];
  float k[1][D];
  float q[1][D];
  float v[1][D];
  float o[D];
  float beta[4];
};

template <int W>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs A) {
  __shared__ DecodeLds L;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int H = A.n_heads;
  const int b = blockIdx.x / H;
  const int h = blockIdx.x - b * H;
  const int slot = A.slot_idx[b];
  if (slot < 0 || slot >= A.n_slots) return;  // whole workgroup together
  const int r0 = 16 * (lane & 7);
  const int col0 = 32 * wave + 4 * (lane >> 3);
  const size_t unit = ((size_t)slot * A.n_layers + A.layer) * H + h;
  float S[16][4];
  load_state(S, A.state_pool + unit * D * D, r0, col0);  // in flight during the prologue

  const int64_t HC = (int64_t)H * D;
  const size_t row = (size_t)b * H + h;  // the token's (request, head) row
  // wave 3, lanes 0..15: the norm's gate and weights, fetched now so the loads overlap the prologue
  const int s16 = lane & 15, wq = s16 >> 2, qq = s16 & 3;
  const int ca = 32 * wq + 4 * qq, cb = ca + 16;
  uint2 ga = make_uint2(0u, 0u), gb = make_uint2(0u, 0u);
  float4 wa = make_float4(0.f, 0.f, 0.f, 0.f), wb = wa;
  if (wave == 3 && lane < 16) {
    const uint16_t* grow = A.gate + row * D;
    ga = *reinterpret_cast<const uint2*>(grow + ca);
    gb = *reinterpret_cast<const uint2*>(grow + cb);
    wa = *reinterpret_cast<const float4*>(A.norm_w + ca);
    wb = *reinterpret_cast<const float4*>(A.norm_w + cb);
  }
  // wave 1, lanes 0..31: exp(gk) of the token while wave 0 runs the prologue (the verify kernel's
  // staging: a = exp(gk) with gk = -softplus(g); a * k follows once k is in LDS)
  if (wave == 1 && lane < 32) {
    const int c4 = 4 * lane;
    const float4 g4 = *reinterpret_cast<const float4*>(A.g_raw + row * D + c4);
    const float gk0 = neg_softplus(g4.x), gk1 = neg_softplus(g4.y), gk2 = neg_softplus(g4.z), gk3 = neg_softplus(g4.w);
    *reinterpret_cast<float4*>(&L.a[0][c4]) = make_float4(expf(gk0), expf(gk1), expf(gk2), expf(gk3));
  }
  if (wave == 0 && lane < 48) {
    const int which = lane >> 4, cg = lane & 15;
    const int ch = h * D + 8 * cg;
    const uint16_t* x = which == 0 ? A.xq : which == 1 ? A.xk : A.xv;
    float w[8][W];
    {
      const float4* wp = reinterpret_cast<const float4*>(A.conv_w + ((int64_t)which * HC + ch) * W);
#pragma unroll
      for (int f = 0; f < 2 * W; ++f) {
        const float4 v4 = wp[f];
        const float e[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) w[(4 * f + q) / W][(4 * f + q) % W] = e[q];
      }
    }
    // taps 0 .. W - 2 are the carried rows (row W - 2 the newest), tap W - 1 the token itself
    uint16_t* cs = W > 1 ? A.conv_state + ((int64_t)b * 3 + which) * (W - 1) * HC + ch : nullptr;  // none at W = 1
    const uint4 xr = *reinterpret_cast<const uint4*>(x + row * D + 8 * cg);
    uint4 tr[W > 1 ? W - 1 : 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) tr[j] = *reinterpret_cast<const uint4*>(cs + j * HC);
    float cur[8];
    widen8(xr, cur);
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = w[i][W - 1] * cur[i];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      float tj[8];
      widen8(tr[j], tj);
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = __builtin_fmaf(w[i][j], tj[i], c[i]);
    }
    float u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = c[i] * sigmoid_fast(c[i]);
    {  // q and k: L2 norm over the head's 16 lanes (the v lanes compute it too and ignore it)
      float ss = u[0] * u[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) ss = __builtin_fmaf(u[i], u[i], ss);
      const float r = __builtin_amdgcn_rsqf(row_sum16(ss) + A.qk_eps);
      if (which < 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = u[i] * r;
      }
    }
    // bf16 as the prologue stores it, then widened as the verify kernel stages it
    const uint4 pk = make_uint4(cvt_pk_bf16(u[0], u[1]), cvt_pk_bf16(u[2], u[3]), cvt_pk_bf16(u[4], u[5]),
                                cvt_pk_bf16(u[6], u[7]));
    float rounded[8];
    widen8(pk, rounded);
    float* dst = which == 0 ? &L.q[0][8 * cg] : which == 1 ? &L.k[0][8 * cg] : &L.v[0][8 * cg];
    *reinterpret_cast<float4*>(dst) = make_float4(rounded[0], rounded[1], rounded[2], rounded[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(rounded[4], rounded[5], rounded[6], rounded[7]);
    // the carried rows move one place towards the past; the token becomes the newest (in place: this
    // lane read exactly these channels above)
#pragma unroll
    for (int j = 0; j + 1 < W - 1; ++j) *reinterpret_cast<uint4*>(cs + j * HC) = tr[j + 1];
    if (W > 1) *reinterpret_cast<uint4*>(cs + (W - 2) * HC) = xr;
  }
  if (wave == 0 && lane == 48) L.beta[0] = sigmoid_fast(A.b_raw[row]);
  __syncthreads();
  if (wave == 1 && lane < 32) {  // ak = a * k, as the verify kernel stages it
    const int c4 = 4 * lane;
    const float4 a4 = *reinterpret_cast<const float4*>(&L.a[0][c4]);
    const float4 k4 = *reinterpret_cast<const float4*>(&L.k[0][c4]);
    *reinterpret_cast<float4*>(&L.ak[0][c4]) = make_float4(a4.x * k4.x, a4.y * k4.y, a4.z * k4.z, a4.w * k4.w);
  }
  __syncthreads();
  step_update(S, L, 0, r0, col0);
  float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 q4 = *reinterpret_cast<const float4*>(&L.q[0][r0 + 4 * i4]);
    const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = __builtin_fmaf(qv[ii], S[4 * i4 + ii][j], y[j]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) y[j] = red8(y[j]);
  if ((lane & 7) == 0) {
    const float4 o4 = make_float4(A.scale * y[0], A.scale * y[1], A.scale * y[2], A.scale * y[3]);
    *reinterpret_cast<float4*>(&L.o[col0]) = o4;
    if (A.o) *reinterpret_cast<float4*>(A.o + row * D + col0) = o4;
  }
  store_state(S, A.state_pool + unit * D * D, r0, col0);  // the commit, in place
  __syncthreads();
  if (wave == 3 && lane < 16) {  // the norm kernel's row: lane s holds slice s, sums gathered in slice order
    const f32x4 oa = *reinterpret_cast<const f32x4*>(&L.o[ca]);
    const f32x4 ob = *reinterpret_cast<const f32x4*>(&L.o[cb]);
    const float part = norm_slice_ssq(oa, ob);
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) ss = ss + __shfl(part, k);
    const float rstd = norm_rstd(ss, A.norm_eps);
    *reinterpret_cast<uint2*>(A.y + row * D + ca) = norm_apply4(oa, ga, wa, rstd);
    *reinterpret_cast<uint2*>(A.y + row * D + cb) = norm_apply4(ob, gb, wb, rstd);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch <= 0) return hipSuccess;
  const dim3 grid((unsigned)a.batch * (unsigned)a.n_heads), block(256);
  switch (a.conv_width) {
    case 1: hipLaunchKernelGGL(decode_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(decode_kernel<3>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_kernel<4>, grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL(decode_kernel<5>, grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL(decode_kernel<6>, grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL(decode_kernel<7>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(decode_kernel<8>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kda
