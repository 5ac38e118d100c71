// kda_prologue.hip -- the KDA prologue (the step before the recurrence) in one kernel: the causal
// depthwise short conv of the q, k and v projections with the conv-state carry, SiLU, the per-head L2
// norm of q and k, beta = sigmoid of its logit, gk = -softplus of the decay logit.
//
// Source: Kimi K3 B200 deployment notes (zdszero.github.io), the prefill / decode kernel-fusion items:
// the three short conv1d calls on q, k, v with their SiLU and the conv-state gather become one kernel,
// beta's copy + sigmoid another. The notes give neither the conv width nor the decay-gate formula; the
// readings (the oracle's as well): width W is an argument, tap j of token t reads token t - W + 1 + j
// (the W - 1 tokens before a sequence come from its carried state), q and k are L2-normalised per head
// after the SiLU with eps inside the root, and gk = -softplus(g) (so exp(gk) = sigmoid(-g)).
//
// The sequence of a token is found by a binary search in cu_seqlens; every bound read from device
// memory is clamped, so no value of it makes the kernel address memory outside the buffers.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_prologue.h"

namespace kda {

namespace {

// sequence n of token t: the last n with cu[n] <= t (cu read clamped into [0, T])
__device__ __forceinline__ int seq_of(const int32_t* cu, int n_seq, int64_t T, int64_t t) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t c = min(max((int64_t)cu[mid], (int64_t)0), T);
    if (c <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

constexpr int kStrip = 32;  // tokens per wave

// A wave takes four adjacent heads over a strip of kStrip consecutive tokens; lane 16 r + cg holds
// channels 8 cg .. 8 cg + 7 of head 4 hq + r (16-byte row loads, 1 KB per wave instruction). Per
// projection it loads its 8 W conv weights once and keeps the last W rows, widened to fp32, in a ring
// of W register sets, and the raw rows of the next U tokens in a second ring (U >= 4, a multiple of W,
// so a wave keeps U row loads in flight); the token loop is unrolled by U, so the slot of every tap is a
// compile-time index and nothing moves. Each x row is read once (plus W - 1 halo rows per strip). The strip's
// sequence structure is the same for all lanes: at a sequence start the ring is refilled from that
// sequence's carried state. The q and k norms are DPP row sums over a row's 16 lanes.
template <int W>
__global__ void __launch_bounds__(256) prologue_kernel(PrologueArgs A) {
  constexpr int U = W <= 2 ? 4 : W == 3 ? 6 : W;  // row prefetch distance and unroll, a multiple of W
  const int lane = threadIdx.x & 63;
  const int H = A.n_heads;
  const int n_hq = (H + 3) >> 2;
  const int64_t T = A.total_tokens;
  const int64_t wv = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int64_t strip = wv / n_hq;
  const int hq = (int)(wv - strip * n_hq);
  const int64_t t0 = strip * kStrip;
  if (t0 >= T) return;  // wave-uniform
  const int64_t t1 = min(t0 + kStrip, T);
  const int h_raw = 4 * hq + (lane >> 4);
  const bool act = h_raw < H;  // a row group past the last head repeats it and stores nothing
  const int h = min(h_raw, H - 1);
  const int64_t HC = (int64_t)H * D;
  const int ch = h * D + 8 * (lane & 15);  // the lane's first channel; row p of a projection at + p HC
  const int n0 = seq_of(A.cu_seqlens, A.n_seq, T, t0);
  for (int which = 0; which < 3; ++which) {
    const uint16_t* x = which == 0 ? A.xq : which == 1 ? A.xk : A.xv;
    uint16_t* out = which == 0 ? A.q : which == 1 ? A.k : A.v;
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
    // the row that token q stands for when sequence n (start s) reads it: x[q] inside the sequence,
    // else row q - s + W - 1 of the carried state (in [0, W - 1) because q >= s - W + 1 where it is read)
    auto tap_row = [&](int n, int64_t s, int64_t q) -> uint4 {
      if (q >= s) return *reinterpret_cast<const uint4*>(x + q * HC + ch);
      if (A.state_in)
        return *reinterpret_cast<const uint4*>(A.state_in + (((int64_t)n * 3 + which) * (W - 1) + (q - s + W - 1)) * HC + ch);
      return make_uint4(0u, 0u, 0u, 0u);
    };
    float R[W][8];  // R[(p - t0 - a) mod W] = row of token p - a, for the token p being computed and a < W
    int n = n0;
    int64_t s = min(max((int64_t)A.cu_seqlens[n], (int64_t)0), t0);
    int64_t e = n + 1 < A.n_seq ? min(max((int64_t)A.cu_seqlens[n + 1], t0 + 1), T) : T;  // next start, > t0
    // the rows before t0 (ages 1 .. W - 1 at the first token, which sits in slot 0)
#pragma unroll
    for (int a = 1; a < W; ++a) widen8(tap_row(n, s, t0 - a), R[W - a]);
    uint4 pre[U];  // raw rows of the next U tokens, token p in slot (p - t0) mod U
#pragma unroll
    for (int d = 0; d < U; ++d)
      if (t0 + d < t1) pre[d] = *reinterpret_cast<const uint4*>(x + (t0 + d) * HC + ch);
    for (int64_t pb = t0; pb < t1; pb += U) {
#pragma unroll
      for (int kk = 0; kk < U; ++kk) {
        const int64_t p = pb + kk;
        const int k = kk % W;  // ring slot of token p
        if (p < t1) {  // wave-uniform
          widen8(pre[kk], R[k]);
          if (p + U < t1) pre[kk] = *reinterpret_cast<const uint4*>(x + (p + U) * HC + ch);
          if (p >= e) {  // p starts a later sequence: find it, refill the older slots from its state
            n = seq_of(A.cu_seqlens, A.n_seq, T, p);
            s = min(max((int64_t)A.cu_seqlens[n], (int64_t)0), p);
            e = n + 1 < A.n_seq ? min(max((int64_t)A.cu_seqlens[n + 1], p + 1), T) : T;
#pragma unroll
            for (int a = 1; a < W; ++a) widen8(tap_row(n, s, p - a), R[(k - a + W) % W]);
          }
          float c[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) c[i] = w[i][W - 1] * R[k][i];
#pragma unroll
          for (int j = 0; j < W - 1; ++j) {  // tap j reads token p - (W - 1) + j
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = __builtin_fmaf(w[i][j], R[(k + 1 + j) % W][i], c[i]);
          }
          float u[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) u[i] = c[i] * sigmoid_fast(c[i]);
          if (which < 2) {
            float ss = u[0] * u[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) ss = __builtin_fmaf(u[i], u[i], ss);
            const float r = __builtin_amdgcn_rsqf(row_sum16(ss) + A.eps);
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = u[i] * r;
          }
          if (act)
            *reinterpret_cast<uint4*>(out + p * HC + ch) = make_uint4(cvt_pk_bf16(u[0], u[1]), cvt_pk_bf16(u[2], u[3]),
                                                                  cvt_pk_bf16(u[4], u[5]), cvt_pk_bf16(u[6], u[7]));
        }
      }
    }
  }
  // the gates, elementwise over the strip
#pragma unroll 4
  for (int64_t p = t0; p < t1; ++p) {
    const float* gp = A.g_raw + p * HC + ch;
    float* gkp = A.gk + p * HC + ch;
    const float4 ga = *reinterpret_cast<const float4*>(gp);
    const float4 gb = *reinterpret_cast<const float4*>(gp + 4);
    if (act) {
      *reinterpret_cast<float4*>(gkp) = make_float4(neg_softplus(ga.x), neg_softplus(ga.y), neg_softplus(ga.z), neg_softplus(ga.w));
      *reinterpret_cast<float4*>(gkp + 4) = make_float4(neg_softplus(gb.x), neg_softplus(gb.y), neg_softplus(gb.z), neg_softplus(gb.w));
    }
  }
  // beta: the 16 lanes of head 4 hq + r take 16 tokens of the strip per pass
  for (int64_t p = t0 + (lane & 15); p < t1; p += 16)
    if (act) A.beta[p * H + h] = sigmoid_fast(A.b_raw[p * H + h]);
}

// the carried state after the batch: row r of (n, which) = token e - (W - 1) + r of the sequence, or,
// for a sequence shorter than W - 1, the older rows of the state it came with (zeros without one)
__global__ void __launch_bounds__(256) prologue_state_kernel(PrologueArgs A) {
  const int64_t HC = (int64_t)A.n_heads * D;
  const int64_t per_row = HC / 2;  // bf16 pairs per row
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int W = A.conv_width;
  const int64_t rows = (int64_t)A.n_seq * 3 * (W - 1);
  if (idx >= rows * per_row) return;
  const int64_t row = idx / per_row, e2 = idx - row * per_row;
  const int r = (int)(row % (W - 1));
  const int which = (int)((row / (W - 1)) % 3);
  const int n = (int)(row / (3 * (W - 1)));
  const int64_t s = min(max((int64_t)A.cu_seqlens[n], (int64_t)0), A.total_tokens);
  const int64_t e = min(max((int64_t)A.cu_seqlens[n + 1], s), A.total_tokens);
  const int64_t p = e - (W - 1) + r;
  const uint16_t* xs[3] = {A.xq, A.xk, A.xv};
  uint32_t v = 0u;
  if (p >= s) {
    v = *reinterpret_cast<const uint32_t*>(xs[which] + p * HC + 2 * e2);
  } else if (A.state_in) {  // p - s + W - 1 = r - (e - s) + ... in [0, W - 1)
    v = *reinterpret_cast<const uint32_t*>(A.state_in + (((int64_t)n * 3 + which) * (W - 1) + (p - s + W - 1)) * HC + 2 * e2);
  }
  *reinterpret_cast<uint32_t*>(A.state_out + row * HC + 2 * e2) = v;
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream) {
  if (a.total_tokens > 0) {
    const int64_t waves = (a.total_tokens + kStrip - 1) / kStrip * ((a.n_heads + 3) / 4);
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    switch (a.conv_width) {
      case 1: hipLaunchKernelGGL(prologue_kernel<1>, grid, block, 0, stream, a); break;
      case 2: hipLaunchKernelGGL(prologue_kernel<2>, grid, block, 0, stream, a); break;
      case 3: hipLaunchKernelGGL(prologue_kernel<3>, grid, block, 0, stream, a); break;
      case 4: hipLaunchKernelGGL(prologue_kernel<4>, grid, block, 0, stream, a); break;
      case 5: hipLaunchKernelGGL(prologue_kernel<5>, grid, block, 0, stream, a); break;
      case 6: hipLaunchKernelGGL(prologue_kernel<6>, grid, block, 0, stream, a); break;
      case 7: hipLaunchKernelGGL(prologue_kernel<7>, grid, block, 0, stream, a); break;
      case 8: hipLaunchKernelGGL(prologue_kernel<8>, grid, block, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.state_out && a.conv_width > 1 && a.n_seq > 0) {
    const int64_t elems = (int64_t)a.n_seq * 3 * (a.conv_width - 1) * a.n_heads * D / 2;
    hipLaunchKernelGGL(prologue_state_kernel, dim3((unsigned)((elems + 255) / 256)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace kda
