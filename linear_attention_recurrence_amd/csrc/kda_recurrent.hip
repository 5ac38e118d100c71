// kda_recurrent.hip -- token-by-token KDA kernels on the fp32 vector ALU (gfx950):
// the speculative verify (one launch per layer) and the ReplaySSM fold (one
// launch over every layer and head).
//
// Sources: "SGLang and Miles Add Day-0 Support for Kimi K3" (LMSYS blog),
// section "ReplaySSM: raw-input replay for the KDA state" -- verify reads the
// committed checkpoint and never writes it and stores each step's raw inputs
// (v, k, gk, beta); the fold replays only the accepted prefix in place with
// the stored gate values and is a verbatim clone of the verify recurrence
// (same tiles, same reduction order), bit-identical to the recurrent commit.
// Kimi K3 B200 deployment notes (zdszero.github.io), section "DSPARK and KDA
// state": the per-slot ring of (v, k, gate, beta) with a power-of-two length.
//
// Both kernels run the SAME step function with the SAME lane -> (row, column)
// ownership and the same reduction order; every product and sum is an
// explicit fmaf / mul / add (the file is built with -ffp-contract=off), and
// the decay comes from the same expf of the same stored fp32 gk. That is what
// makes the fold bit-identical to verify's commit.
//
// Work decomposition: one 256-thread workgroup per (request, head) for verify
// and per (request, layer, head) for fold. The fp32 state S[128][128] lives in
// registers: wave w, lane l owns rows 16*(l&7) .. +15 and columns
// 32*w + 4*(l>>3) .. +3 (64 floats). Sums over the key channel are a
// sequential FMA chain over the thread's 16 rows, then a butterfly over the
// eight lanes l&7 that share the columns (DPP quad_perm x2, row_half_mirror).
// A column of S evolves independently of the others given the key-side values,
// and each 32-column block is one wave's: so when there are few (request, head)
// pairs (single-request decode: 96 heads for 256 compute units) verify runs one
// 64-thread workgroup per (request, head, 32-column block), each wave computing
// its columns exactly as it would inside the 256-thread workgroup (same lanes,
// same reduction order), so outputs and commits are bit for bit the same.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_step.h"

namespace kda {

// load 4 consecutive q/k/v elements as fp32 (bf16 widened exactly)
template <bool F32>
__device__ __forceinline__ float4 load4(const void* base, size_t idx) {
  if constexpr (F32) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
  } else {
    const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return make_float4(bf2f(r.x & 0xffffu), bf2f(r.x >> 16), bf2f(r.y & 0xffffu), bf2f(r.y >> 16));
  }
}

template <bool F32, bool RING, bool SPLIT>
__global__ void __launch_bounds__(256) verify_kernel(VerifyArgs A) {
  __shared__ StepLds L;
  constexpr int NT = SPLIT ? 64 : 256;  // threads per workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = SPLIT ? (int)(blockIdx.x & 3) : tid >> 6;       // the 32-column block
  const int ub = SPLIT ? (int)(blockIdx.x >> 2) : (int)blockIdx.x;  // (request, head)
  const int r0 = 16 * (lane & 7);
  const int col0 = 32 * wave + 4 * (lane >> 3);
  const int b = ub / A.n_heads;
  const int h = ub - b * A.n_heads;
  const int slot = A.slot_idx[b];
  if (slot < 0 || slot >= A.n_slots) return;  // whole workgroup skips together
  const size_t unit = ((size_t)slot * A.n_layers + A.layer) * A.n_heads + h;

  // the state slice first: the commit length and the ring start are read after its loads are
  // issued, so that their memory latency is not paid before the state's
  float S[16][4];
  load_state(S, A.state_pool + unit * D * D, r0, col0);
  int commit_n = 0;
  if (A.commit_len && A.commit_pool) {
    commit_n = A.commit_len[b];
    commit_n = commit_n < 0 ? 0 : (commit_n > A.n_tok ? A.n_tok : commit_n);
  }
  const int rstart = (RING && A.ring_start) ? A.ring_start[b] : 0;

  for (int t0 = 0; t0 < A.n_tok; t0 += TB) {
    const int nb = (A.n_tok - t0) < TB ? (A.n_tok - t0) : TB;
    __syncthreads();  // the previous batch is no longer read
    for (int x = tid; x < 32 * TB; x += NT) {  // one pass with 256 threads
      const int tt = x >> 5, c4 = (x & 31) * 4;
      if (tt < nb) {
        const size_t row = ((size_t)b * A.n_tok + t0 + tt) * A.n_heads + h;
        const size_t e = row * D + c4;
        const float4 g4 = *reinterpret_cast<const float4*>(A.gk + e);
        const float4 k4 = load4<F32>(A.k, e);
        const float4 q4 = load4<F32>(A.q, e);
        const float4 v4 = load4<F32>(A.v, e);
        const float a0 = expf(g4.x), a1 = expf(g4.y), a2 = expf(g4.z), a3 = expf(g4.w);
        *reinterpret_cast<float4*>(&L.a[tt][c4]) = make_float4(a0, a1, a2, a3);
        *reinterpret_cast<float4*>(&L.ak[tt][c4]) = make_float4(a0 * k4.x, a1 * k4.y, a2 * k4.z, a3 * k4.w);
        *reinterpret_cast<float4*>(&L.k[tt][c4]) = k4;
        *reinterpret_cast<float4*>(&L.q[tt][c4]) = q4;
        *reinterpret_cast<float4*>(&L.v[tt][c4]) = v4;
        const float beta = A.beta[row];
        if (c4 == 0) L.beta[tt] = beta;
        if (RING && (!SPLIT || wave == 0)) {
          // raw inputs, bit for bit, into ring position (start + t) & (len - 1)
          const int pos = (rstart + t0 + tt) & (A.ring_len - 1);
          const size_t rrow = unit * A.ring_len + pos;
          const size_t re = rrow * D + c4;
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(A.ring_k) + re) =
              *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(A.k) + e);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(A.ring_v) + re) =
              *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(A.v) + e);
          *reinterpret_cast<float4*>(A.ring_gk + re) = g4;
          if (c4 == 0) A.ring_beta[rrow] = beta;
        }
      }
    }
    __syncthreads();
    for (int tt = 0; tt < nb; ++tt) {
      step_update(S, L, tt, r0, col0);
      // readout o_t = scale * S^T q_t from the updated state
      float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 q4 = *reinterpret_cast<const float4*>(&L.q[tt][r0 + 4 * i4]);
        const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = __builtin_fmaf(qv[ii], S[4 * i4 + ii][j], y[j]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = red8(y[j]);
      if ((lane & 7) == 0) {
        const size_t orow = ((size_t)b * A.n_tok + t0 + tt) * A.n_heads + h;
        *reinterpret_cast<float4*>(A.o + orow * D + col0) =
            make_float4(A.scale * y[0], A.scale * y[1], A.scale * y[2], A.scale * y[3]);
      }
      if (t0 + tt + 1 == commit_n) store_state(S, A.commit_pool + unit * D * D, r0, col0);
    }
  }
}

__global__ void __launch_bounds__(256) fold_kernel(FoldArgs A) {
  __shared__ StepLds L;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r0 = 16 * (lane & 7);
  const int col0 = 32 * wave + 4 * (lane >> 3);
  const int h = blockIdx.x % A.n_heads;
  const int bl = blockIdx.x / A.n_heads;
  const int l = bl % A.n_layers;
  const int b = bl / A.n_layers;
  const int slot = A.slot_idx[b];
  if (slot < 0 || slot >= A.n_slots) return;
  int n = A.accepted_len[b];
  const int nmax = A.ring_len >> 1;
  n = n < 0 ? 0 : (n > nmax ? nmax : n);
  if (n == 0) return;  // rejected everything: the committed state stays as is
  const int rstart = A.ring_start ? A.ring_start[b] : 0;
  const size_t unit = ((size_t)slot * A.n_layers + l) * A.n_heads + h;

  float S[16][4];
  load_state(S, A.state_pool + unit * D * D, r0, col0);
  for (int t0 = 0; t0 < n; t0 += TB) {
    const int nb = (n - t0) < TB ? (n - t0) : TB;
    __syncthreads();
    {
      const int tt = tid >> 5, c4 = (tid & 31) * 4;
      if (tt < nb) {
        const int pos = (rstart + t0 + tt) & (A.ring_len - 1);
        const size_t rrow = unit * A.ring_len + pos;
        const size_t re = rrow * D + c4;
        stage_entry(L, tt, c4, *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(A.ring_k) + re),
                    *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(A.ring_v) + re),
                    *reinterpret_cast<const float4*>(A.ring_gk + re), A.ring_beta[rrow]);
      }
    }
    __syncthreads();
    for (int tt = 0; tt < nb; ++tt) step_update(S, L, tt, r0, col0);
  }
  store_state(S, A.state_pool + unit * D * D, r0, col0);
}

hipError_t launch_verify(const VerifyArgs& a, bool f32, hipStream_t stream) {
  if (verify_chunk_eligible(a, f32)) return launch_verify_chunk(a, stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const long units = (long)a.batch * a.n_heads;
  const bool ring = a.ring_k != nullptr;
  if (units < 2L * prefill_max_grid(dev)) {  // fewer than two (request, head) pairs per CU: split columns
    const dim3 grid((unsigned)(4 * units)), block(64);
    if (f32) hipLaunchKernelGGL((verify_kernel<true, false, true>), grid, block, 0, stream, a);
    else if (ring) hipLaunchKernelGGL((verify_kernel<false, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((verify_kernel<false, false, true>), grid, block, 0, stream, a);
  } else {
    const dim3 grid((unsigned)units), block(256);
    if (f32) hipLaunchKernelGGL((verify_kernel<true, false, false>), grid, block, 0, stream, a);
    else if (ring) hipLaunchKernelGGL((verify_kernel<false, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((verify_kernel<false, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_fold(const FoldArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.batch * (unsigned)a.n_layers * (unsigned)a.n_heads), block(256);
  hipLaunchKernelGGL(fold_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
