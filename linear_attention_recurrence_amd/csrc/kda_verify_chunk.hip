// kda_verify_chunk.hip -- speculative verify of up to 16 draft tokens in chunked
// form on the gfx950 matrix cores.
//
// Sources: "SGLang and Miles Add Day-0 Support for Kimi K3" (LMSYS blog),
// section "ReplaySSM: raw-input replay for the KDA state" -- verify reads the
// committed state without writing it and records each step's raw inputs
// (v, k, gk, beta) for the fold. Kimi K3 B200 deployment notes
// (zdszero.github.io), section "DSPARK and KDA state" -- the per-slot ring.
//
// Verify needs the outputs of every draft token but never the state after
// them (the fold produces that later from the ring), so the T tokens are one
// chunk of the chunked form, with S0 the committed state and
// G_t = sum_{tau<=t} gk_tau from the first draft token:
//   A[i][j] = beta_i sum_c (k_ic e^{G_ic}) (k_jc e^{-G_jc})   (j < i)
//   P[t][i] =        sum_c (q_tc e^{G_tc}) (k_ic e^{-G_ic})   (i <= t)
//   R = diag(beta) (V - Kt S0),  W = (I + A)^-1 R,  O = scale (Qt S0 + P W)
// with Kt = k e^G and Qt = q e^G. The factors e^{-G} grow with the decay
// summed over the window, which stays in fp32/bf16 range while that sum is at
// most 80 per key channel. A unit whose window decays more in some channel
// (gk = -inf included) forms A and P pairwise instead, each entry in fp32 from
// the exponential of the decay summed between its two tokens, so the path is
// exact for any gk <= 0; decays are clamped at e^-110 per token (0 in fp32).
//
// Precision follows the prefill kernel: A and P from bf16 MFMAs with the
// q e^G and k e^{-G} factors split into bf16 hi + lo (k e^G single); the state
// products on fp16 MFMAs with R and W as fp16 hi + lo; fp32 accumulation.
// A call that also asks for the recurrent commit takes the token-by-token
// kernel instead, whose arithmetic the fold replays bit for bit.
//
// Work decomposition: a persistent grid of 256-thread workgroups, two per CU,
// each taking (request, head) units in turn and prefetching the next unit's
// state slice and inputs into registers while it computes the current one.
// Wave w stages its 128 x 32 column slice of S0 as fp16 in LDS (coalesced
// 16-byte loads; on the plain and trimmed paths after the unit's key side, on
// the fused path after the fold) and reads it back transposed
// (ds_read_b64_tr_b16) as MFMA operands.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_step.h"

namespace kda {

namespace {

constexpr int VT = 16;   // tokens per call on this path (padded)
constexpr float kMinDecay = -110.f;        // per-token log-decay clamp: e^-110 is 0 in fp32
constexpr float kMaxWindowDecay = 80.f;    // factor form's range: sum(-gk) over the window per channel
constexpr int TV = 136;  // operand row stride (16-bit elements; 128 + 8 pad)
constexpr int PS = 24;   // 16x16 fp16 rows (+8 pad)

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit data format: range-checked by num_records
constexpr int kStream = 2;             // cache policy of the output stores: non-temporal (written once, read by later launches)
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int NT>
struct alignas(16) VerifyLds {
  uint16_t sh[4][D][32];   // per wave: fp16 S0[c][32w + j]
  union {
    struct {
      uint16_t kt[VT][TV];     // fp16 k e^G, rows t
      uint16_t qt[VT][TV];     // fp16 q e^G
      uint16_t rk[VT][TV];     // bf16 k e^G
      uint16_t rqh[VT][TV];    // bf16 q e^G, hi
      uint16_t rql[VT][TV];    //                lo
      uint16_t ckh[VT][TV];    // bf16 k e^{-G}, hi
      uint16_t ckl[VT][TV];    //                 lo
    };
    FoldLds fold;  // fused fold: the previous window's entries, staged before the rows are formed
  };
  uint16_t v[VT][D];       // bf16 v rows
  uint16_t xh[VT][PS];     // fp16 X = (I + A)^-1, rows t
  uint16_t ph[VT][PS];     // fp16 P, rows t
  float am[VT][20];        // A rows (fp32) for the solve
  float beta[VT];
  int exact;               // this unit's window decays beyond the factor form's range
  alignas(16) uint16_t kin[NT][D];  // raw k, q (bf16) and gk rows of the window; after the decay factors,
  uint16_t qin[NT][D];              // the four waves' A and P partials (8 KB) on the fast path
  float gin[NT][D];
};

__device__ __forceinline__ uint2 lds8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
// a range-checked buffer over `bytes` bytes at p, read only here (an empty range reads zeros)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t read_range(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kBufWord3);
}
// A wave-uniform 32-bit read through the scalar data cache. Plain loads of these
// indices are emitted as vector loads, and waiting for one of those waits for every
// older vector memory operation of the wave (prefetches and stores included).
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}
__device__ __forceinline__ uint2 lds_tr(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}
__device__ __forceinline__ f16x8 as_f16x8(uint2 a, uint2 b) {
  return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// permuted 32-wide reduction step: row elements {4g..4g+3} then {16+4g..16+4g+3}
__device__ __forceinline__ f16x8 perm_h(const uint16_t* row, int g) { return as_f16x8(lds8(row + 4 * g), lds8(row + 16 + 4 * g)); }
__device__ __forceinline__ bf16x8 perm_b(const uint16_t* row, int g) { return as_bf16x8(lds8(row + 4 * g), lds8(row + 16 + 4 * g)); }
__device__ __forceinline__ f32x4 mfma_h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_h16(const f16x4& a, const f16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint16_t h16(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
// fp16 hi + lo: hi = f16(x), lo = f16(x - hi), the exact remainder formed by one mixed-precision
// FMA that takes the packed fp16 hi as its operand; mone is -1.0f held in a register (with a
// literal the compiler folds the FMA back into a subtraction)
__device__ __forceinline__ void split_h4(const f32x4& a, f16x4& hi, f16x4& lo, float mone) {
  f16x2 h0 = {(_Float16)a[0], (_Float16)a[1]}, h1 = {(_Float16)a[2], (_Float16)a[3]};
  asm("" : "+v"(h0), "+v"(h1));
  hi = f16x4{h0[0], h0[1], h1[0], h1[1]};
  lo = f16x4{(_Float16)__builtin_fmaf((float)h0[0], mone, a[0]), (_Float16)__builtin_fmaf((float)h0[1], mone, a[1]),
             (_Float16)__builtin_fmaf((float)h1[0], mone, a[2]), (_Float16)__builtin_fmaf((float)h1[1], mone, a[3])};
}

}  // namespace

// Persistent: each workgroup walks units u = blockIdx.x, + gridDim.x, ...; the
// next unit's committed state and raw inputs are loaded into registers while
// the current one computes. NT is the padded window (8 or 16 tokens); with
// RAGGED each request has its own window (rows cu_tok[b] .. cu_tok[b + 1] - 1,
// clamped), otherwise every request has n_tok tokens at rows b n_tok + t. Every
// global store of a unit is unconditional (the outputs of padded tokens are
// dropped by the buffer range check), so the compiler's wait before the next
// unit's first use of its prefetched registers leaves the stores in flight.
template <bool RING, int NT, bool FOLD, bool RAGGED>
__global__ void __launch_bounds__(256, 2) verify_chunk_kernel(VerifyArgs A) {
  __shared__ VerifyLds<NT> L;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, lr = lane & 15;
  const int H = A.n_heads;
  const int T = A.n_tok;  // 1 .. NT (with RAGGED: the bound on every window)
  const int n_units = A.batch * H;
  constexpr int NH = NT / 2;              // tokens per input thread
  const int c = tid & (D - 1);            // input thread: channel c ...
  const int t0 = NH * (tid >> 7);         // ... of tokens t0 .. t0 + NH - 1

  // rows NT .. 15 of the operand matrices stay zero for the whole launch (MFMA tiles are 16 tall)
  if constexpr (NT < VT) {
    for (int e = tid; e < (VT - NT) * D; e += 256) {
      const int t = NT + e / D, cc = e % D;
      L.kt[t][cc] = 0; L.qt[t][cc] = 0; L.rk[t][cc] = 0; L.rqh[t][cc] = 0; L.rql[t][cc] = 0;
      L.ckh[t][cc] = 0; L.ckl[t][cc] = 0; L.v[t][cc] = 0;
    }
    if (tid < VT - NT) L.beta[NT + tid] = 0.f;
  }

  // unit u = (request b, head h); a request without a valid slot still runs (on state of slot 0)
  // but every store it makes is dropped by an empty buffer range
  auto unit_of = [&](int u, int& b, int& h, size_t& unit) -> bool {
    // uniform values kept in scalar registers, so that the index loads are scalar ones and never
    // wait behind the vector memory queue
    b = __builtin_amdgcn_readfirstlane(u / H);
    h = __builtin_amdgcn_readfirstlane(u - b * H);
    const int slot = sload_i32(A.slot_idx + b);
    const bool valid = slot >= 0 && slot < A.n_slots;
    unit = ((size_t)(valid ? slot : 0) * A.n_layers + A.layer) * H + h;
    return valid;
  };
  // prefetched registers of one unit: this wave's 128 x 32 state slice (16-byte loads, 8 rows per
  // instruction) and 4 channels c4 .. c4+3 of tokens ti and ti + 8 (tokens past the window re-read
  // the last one)
  constexpr int NI = NT / 8;
  const int ti = tid >> 5, c4 = 4 * (tid & 31);
  // the fold's ownership of the state (the recurrence step's): rows r0 .. r0 + 15, columns col0 .. col0 + 3
  const int r0 = 16 * (lane & 7), col0 = 32 * wave + 4 * (lane >> 3);
  float4 sv[16];
  uint2 pk[NI], pq[NI], pv[NI];
  float4 pg[NI];
  float pb[NI];
  uint2 fk, fv;  // fused fold: entry ti of the previous window (channels c4 .. c4 + 3)
  float4 fg;
  float fb;
  // entries of the previous window to fold for request b (clamped like the fold's)
  auto fold_n = [&](int b) {
    const int n = sload_i32(A.fold_len + b), nmax = A.ring_len >> 1;
    return n < 0 ? 0 : (n > nmax ? nmax : n);
  };
  // loads i0 .. i1 - 1 of the 16 that bring in the state slice of a unit (in the fold's ownership
  // on the fused path). The plain path stages a unit's slice into LDS only when its state
  // products need it, after the key side (decay factors, A, P, X), which does not: the first
  // unit's slice arrives while that work runs, and the next unit's slice is issued at once into
  // the registers the staging frees. The fused path folds the state first, so it stages early and
  // issues the next slice in three pieces between its compute phases (all 16 at once there fill
  // the memory queue and stall the issuing wave with this unit's compute still to do).
  // The loads go through a buffer range over the unit's state, empty when there is no next unit:
  // the same instructions are issued and return zeros without touching memory.
  auto state_range = [&](size_t unit, bool live) {
    return read_range(A.state_pool + unit * D * D, live ? D * D * 4 : 0);
  };
  auto prefetch_state = [&](__amdgpu_buffer_rsrc_t srs, int i0, int i1) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i >= i0 && i < i1) {
        const int off = FOLD ? ((r0 + i) * D + col0) * 4 : ((8 * i + (lane >> 3)) * D + 32 * wave + 4 * (lane & 7)) * 4;
        sv[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(srs, off, 0, 0));
      }
  };
  constexpr int kPiece1 = 4, kPiece2 = 10;  // fused path: loads issued after staging, after the decay factors, after A and P
  // the window of request b: its first input row and its length tn <= T. Ragged bounds are
  // clamped into [0, total_tok] (the host passes total_tok >= 1), so a row index never leaves
  // the tensors whatever cu_tok holds
  auto window = [&](int b, size_t& first, int& tn) {
    if constexpr (RAGGED) {
      const int s = min(max(sload_i32(A.cu_tok + b), 0), A.total_tok);
      const int e = min(max(sload_i32(A.cu_tok + b + 1), s), A.total_tok);
      first = (size_t)s;
      tn = min(e - s, T);
    } else {
      first = (size_t)b * T;
      tn = T;
    }
  };
  // the raw inputs of a unit (and the entries to fold on the fused path), through buffer ranges
  // over the unit's rows that are empty when there is no such unit (live false) or no window:
  // the loads are issued all the same and return zeros without touching memory
  auto prefetch_inputs = [&](int b, int h, size_t unit, bool live) {
    if constexpr (FOLD) {
      // entries past the window re-read its last one (or its first, for an empty window)
      const int n = fold_n(b), fs = A.fold_start ? sload_i32(A.fold_start + b) : 0;
      const int pos = (fs + min(ti, max(n - 1, 0))) & (A.ring_len - 1);
      const int nrow = live ? A.ring_len : 0;
      const size_t rbase = unit * A.ring_len;
      const int re = pos * D + c4;
      fk = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
               read_range(static_cast<const uint16_t*>(A.ring_k) + rbase * D, nrow * D * 2), 2 * re, 0, 0));
      fv = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
               read_range(static_cast<const uint16_t*>(A.ring_v) + rbase * D, nrow * D * 2), 2 * re, 0, 0));
      fg = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
               read_range(A.ring_gk + rbase * D, nrow * D * 4), 4 * re, 0, 0));
      fb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
               read_range(A.ring_beta + rbase, nrow * 4), 4 * pos, 0, 0));
    }
    size_t first;
    int tn;
    window(b, first, tn);
    // rows first .. first + tn - 1 of head h: row t at (first + t) * H + h
    const size_t row0 = first * H + h;
    const uint32_t span = (live && tn > 0) ? ((uint32_t)(tn - 1) * H + 1) * D : 0u;  // elements
    const __amdgpu_buffer_rsrc_t krs = read_range(static_cast<const uint16_t*>(A.k) + row0 * D, 2 * span);
    const __amdgpu_buffer_rsrc_t qrs = read_range(static_cast<const uint16_t*>(A.q) + row0 * D, 2 * span);
    const __amdgpu_buffer_rsrc_t vrs = read_range(static_cast<const uint16_t*>(A.v) + row0 * D, 2 * span);
    const __amdgpu_buffer_rsrc_t grs = read_range(A.gk + row0 * D, 4 * span);
    const __amdgpu_buffer_rsrc_t brs = read_range(A.beta + row0, 4 * (span / D));
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      // tokens past the window re-read its last row
      const int t = min(ti + 8 * n, max(tn - 1, 0));
      const int e = t * H * D + c4;
      pk[n] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(krs, 2 * e, 0, 0));
      pq[n] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(qrs, 2 * e, 0, 0));
      pv[n] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vrs, 2 * e, 0, 0));
      pg[n] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(grs, 4 * e, 0, 0));
      pb[n] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(brs, 4 * t * H, 0, 0));
    }
  };
  if (blockIdx.x < (unsigned)n_units) {
    int b, h;
    size_t unit;
    unit_of(blockIdx.x, b, h, unit);
    prefetch_inputs(b, h, unit, true);
    prefetch_state(state_range(unit, true), 0, 16);
    // The same stores as the end of an iteration, into empty ranges (dropped): the loop is
    // then entered with the same pattern of outstanding memory operations from both sides,
    // and the compiler's wait for the prefetched registers need not drain the stores.
    const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(A.o, 0, 0, kBufWord3);
    const u32x4 z = {0u, 0u, 0u, 0u};
    if constexpr (RING) {
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, none, 0, 0, kStream);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, none, 0, 0, kStream);
        __builtin_amdgcn_raw_buffer_store_b128(z, none, 0, 0, kStream);
        __builtin_amdgcn_raw_buffer_store_b32(0u, none, 0, 0, kStream);
      }
    }
    __builtin_amdgcn_raw_buffer_store_b128(z, none, 0, 0, kStream);
    __builtin_amdgcn_raw_buffer_store_b128(z, none, 0, 0, kStream);
  }

  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    int b, h;
    size_t unit;
    const bool ok = unit_of(u, b, h, unit);  // wave-uniform
    if constexpr (FOLD) {
      // the two workgroups sharing a CU drift apart (the older one's waves win the issue
      // arbitration), and the one behind would run its last units alone: a wave's priority is the
      // number of units its workgroup has left after this one, so the one behind issues first.
      // (Worth 1.8 % on the fused path; with the plain path's late state staging it no longer
      // helps the plain verify and costs the trimmed one 0.8 %, so those keep one priority.)
      const int left = (n_units - 1 - u) / (int)gridDim.x;
      if (left >= 3) __builtin_amdgcn_s_setprio(3);
      else if (left == 2) __builtin_amdgcn_s_setprio(2);
      else if (left == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();                         // the previous unit's LDS readers are done
    float S[16][4];                          // fused fold: the state, in the recurrence step's ownership
    int fn = 0;                              // entries to fold
    if (tid == 0) L.exact = 0;               // set below by any channel beyond the factor form's range
    if constexpr (FOLD) {
#pragma unroll
      for (int i = 0; i < 16; ++i) { S[i][0] = sv[i].x; S[i][1] = sv[i].y; S[i][2] = sv[i].z; S[i][3] = sv[i].w; }
      fn = fold_n(b);
      if (ti < fn) stage_entry(L.fold, ti, c4, fk, fv, fg, fb);
    }
    // raw inputs: staging rows, v and beta for the chain, and the ring (bit copies; tokens past
    // the window rewrite the last entry with the same bits)
    const int rstart = (RING && A.ring_start) ? sload_i32(A.ring_start + b) : 0;
    size_t first;  // this request's window: input rows first .. first + tn - 1
    int tn;
    window(b, first, tn);
    __amdgpu_buffer_rsrc_t rk_rs, rv_rs, rg_rs, rb_rs;  // this unit's ring rows (empty without a slot or a window)
    if constexpr (RING) {
      const int nrow = (ok && tn > 0) ? A.ring_len : 0;
      rk_rs = __builtin_amdgcn_make_buffer_rsrc(static_cast<uint16_t*>(A.ring_k) + unit * A.ring_len * D, 0, nrow * D * 2, kBufWord3);
      rv_rs = __builtin_amdgcn_make_buffer_rsrc(static_cast<uint16_t*>(A.ring_v) + unit * A.ring_len * D, 0, nrow * D * 2, kBufWord3);
      rg_rs = __builtin_amdgcn_make_buffer_rsrc(A.ring_gk + unit * A.ring_len * D, 0, nrow * D * 4, kBufWord3);
      rb_rs = __builtin_amdgcn_make_buffer_rsrc(A.ring_beta + unit * A.ring_len, 0, nrow * 4, kBufWord3);
    }
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int t = ti + 8 * n;
      const bool ok_t = t < tn;
      *reinterpret_cast<uint2*>(&L.kin[t][c4]) = pk[n];
      *reinterpret_cast<uint2*>(&L.qin[t][c4]) = pq[n];
      *reinterpret_cast<float4*>(&L.gin[t][c4]) = pg[n];
      *reinterpret_cast<uint2*>(&L.v[t][c4]) = ok_t ? pv[n] : make_uint2(0u, 0u);
      if (c4 == 0) L.beta[t] = ok_t ? pb[n] : 0.f;
      if constexpr (RING) {
        const int pos = (rstart + min(t, tn - 1)) & (A.ring_len - 1);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pk[n]), rk_rs, 2 * (pos * D + c4), 0, kStream);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pv[n]), rv_rs, 2 * (pos * D + c4), 0, kStream);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pg[n]), rg_rs, 4 * (pos * D + c4), 0, kStream);
        // beta is one value per token: only the lane of channel 0 stores it (the others aim past the
        // range and are dropped), instead of 32 lanes storing the same four bytes
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pb[n]), rb_rs, c4 == 0 ? 4 * pos : 0x7ffffff0, 0, kStream);
      }
    }
    // the next unit streams in while this one computes (past the last unit, the same loads into
    // empty ranges, so that every iteration issues the same instructions); the fused fold issues
    // its state after the fold, whose state shares the registers
    int bn, hn;
    size_t unitn;
    const int un = u + (int)gridDim.x;
    const bool more = un < n_units;  // wave-uniform
    unit_of(more ? un : u, bn, hn, unitn);
    prefetch_inputs(bn, hn, unitn, more);
    const __amdgpu_buffer_rsrc_t srs = state_range(unitn, more);
    const size_t row0 = first * H + h;  // input row of token t: row0 + t * H
    __syncthreads();
    if constexpr (FOLD) {
      // the previous window's accepted entries, replayed exactly as the fold does, then the
      // committed state written back in place (dropped by an empty range when the slot is
      // invalid or nothing is folded) and its fp16 copy staged for the verify below
      for (int tt = 0; tt < fn; ++tt) step_update(S, L.fold, tt, r0, col0);
      const __amdgpu_buffer_rsrc_t prs =
          __builtin_amdgcn_make_buffer_rsrc(A.fold_pool + unit * D * D, 0, (ok && fn > 0) ? D * D * 4 : 0, kBufWord3);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(S[i][0]), __float_as_uint(S[i][1]),
                                                     __float_as_uint(S[i][2]), __float_as_uint(S[i][3])},
                                               prs, ((r0 + i) * D + col0) * 4, 0, 0);
        const uint32_t lo = pack2(h16(S[i][0]), h16(S[i][1])), hi = pack2(h16(S[i][2]), h16(S[i][3]));
        *reinterpret_cast<uint2*>(&L.sh[wave][r0 + i][4 * (lane >> 3)]) = make_uint2(lo, hi);
      }
      prefetch_state(srs, 0, kPiece1);
      __syncthreads();
      // the fold's staging shares memory with the operand rows kt, qt, rk and rqh (FoldLds spans
      // 16.4 KB of them): their padding rows NT .. 15, which every MFMA tile reads, must be zero
      // again (a non-finite value there times a zero entry of P would reach O)
      static_assert(sizeof(FoldLds) <= 4 * sizeof(L.kt), "the fold staging must fit in kt, qt, rk and rqh");
      static_assert(offsetof(VerifyLds<NT>, qt) == offsetof(VerifyLds<NT>, kt) + sizeof(L.kt) &&
                        offsetof(VerifyLds<NT>, rqh) == offsetof(VerifyLds<NT>, kt) + 3 * sizeof(L.kt),
                    "kt, qt, rk and rqh are consecutive");
      for (int e = tid; e < 4 * (VT - NT) * (D / 8); e += 256) {
        const int arr = e / ((VT - NT) * (D / 8)), rem = e % ((VT - NT) * (D / 8));
        *reinterpret_cast<uint4*>(&L.kt[0][0] + arr * VT * TV + (NT + rem / (D / 8)) * TV + 8 * (rem % (D / 8))) =
            make_uint4(0u, 0u, 0u, 0u);
      }
    }

    // ---- decay factors of channel c over tokens t0 .. t0 + NH - 1, from the decay summed over
    // the tokens before them
    {
      float gs = 0.f;
      if (t0) {
#pragma unroll
        for (int j = 0; j < NH; ++j) gs += (j < tn) ? __builtin_fmaxf(L.gin[j][c], kMinDecay) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int t = t0 + j;
        const bool ok_t = t < tn;
        const float kv = bf2f(L.kin[t][c]), qv = bf2f(L.qin[t][c]);
        gs += ok_t ? __builtin_fmaxf(L.gin[t][c], kMinDecay) : 0.f;
        const float e = __expf(gs), ie = __expf(-gs);
        const float ke = ok_t ? kv * e : 0.f, qe = ok_t ? qv * e : 0.f, ck = ok_t ? kv * ie : 0.f;
        L.kt[t][c] = h16(ke);
        L.qt[t][c] = h16(qe);
        L.rk[t][c] = f2bf(ke);
        uint16_t hi, lo;
        split_bf16(qe, hi, lo);
        L.rqh[t][c] = hi; L.rql[t][c] = lo;
        split_bf16(ck, hi, lo);
        L.ckh[t][c] = hi; L.ckl[t][c] = lo;
      }
      if (gs < -kMaxWindowDecay) L.exact = 1;  // e^{-G} would leave the range
    }
    if constexpr (FOLD) prefetch_state(srs, kPiece1, kPiece2);
    __syncthreads();

    // ---- A, P and X = (I + A)^-1
    const bool exact = L.exact != 0;  // workgroup-uniform: written before the last barrier
    // A and P partials of one reduction step (32 channels) per wave, kept in the raw rows' space
    // (kin, qin, gin: read only by the decay factors above and by the exact path): [wave][A, P][lane]
    f32x4* part = reinterpret_cast<f32x4*>(&L.kin[0][0]);
    static_assert(offsetof(VerifyLds<NT>, qin) == offsetof(VerifyLds<NT>, kin) + sizeof(L.kin) &&
                      offsetof(VerifyLds<NT>, gin) == offsetof(VerifyLds<NT>, qin) + sizeof(L.qin) &&
                      offsetof(VerifyLds<NT>, kin) % 16 == 0 &&
                      sizeof(L.kin) + sizeof(L.qin) + sizeof(L.gin) >= 4 * 2 * 64 * sizeof(f32x4),
                  "the partials need 8 KB of contiguous, aligned raw-row space");
    if (exact) {
      // pairwise: thread (i, j) forms its entry over the 128 channels, e^{G_ic - G_jc} from the decay
      // summed over tokens j + 1 .. i (tokens past the window only reach rows whose beta is 0)
      const int i = tid >> 4, j = tid & 15;
      float a = 0.f, pp = 0.f;
      if (i < NT && j <= i) {
        for (int cc = 0; cc < D; ++cc) {
          float d = 0.f;
          for (int tt = j + 1; tt <= i; ++tt) d += __builtin_fmaxf(L.gin[tt][cc], kMinDecay);
          const float kje = bf2f(L.kin[j][cc]) * __expf(d);
          a = __builtin_fmaf(bf2f(L.kin[i][cc]), kje, a);
          pp = __builtin_fmaf(bf2f(L.qin[i][cc]), kje, pp);
        }
      }
      L.am[i][j] = (i < NT && j < i) ? a * L.beta[i] : 0.f;
      L.ph[i][j] = (i < NT && j <= i) ? h16(pp) : (uint16_t)0;
    } else {
      const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
      const int s = wave;
      const bf16x8 rk = perm_b(&L.rk[lr][32 * s], g);
      const bf16x8 qh = perm_b(&L.rqh[lr][32 * s], g), ql = perm_b(&L.rql[lr][32 * s], g);
      const bf16x8 ch = perm_b(&L.ckh[lr][32 * s], g), cl = perm_b(&L.ckl[lr][32 * s], g);
      part[(2 * wave) * 64 + lane] = mfma16(rk, cl, mfma16(rk, ch, z4));
      part[(2 * wave + 1) * 64 + lane] = mfma16(ql, ch, mfma16(qh, cl, mfma16(qh, ch, z4)));
    }
    __syncthreads();
    if (wave == 0) {
      if (!exact) {
        // the four waves' partials in wave order; lane (g, lr) holds entries (4g + r, lr)
        f32x4 am = part[lane], pm = part[64 + lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const f32x4 a4 = part[(2 * w) * 64 + lane], p4 = part[(2 * w + 1) * 64 + lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) { am[r] += a4[r]; pm[r] += p4[r]; }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * g + r, j = lr;
          L.am[i][j] = (j < i) ? am[r] * L.beta[i] : 0.f;
          L.ph[i][j] = (j <= i) ? h16(pm[r]) : (uint16_t)0;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      // forward substitution on rows: DPP row g holds columns 4g .. 4g+3 of row i = lr
      float arow[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 a4 = *reinterpret_cast<const float4*>(&L.am[lr][4 * q4]);
        arow[4 * q4] = -a4.x; arow[4 * q4 + 1] = -a4.y; arow[4 * q4 + 2] = -a4.z; arow[4 * q4 + 3] = -a4.w;
      }
      float x[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) x[m] = (4 * g + m == lr) ? 1.f : 0.f;
#define KDA_VSOLVE_STEP(kk)                                                                                   \
      _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                                           \
        const float xk_ = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[m]), 0x150 + (kk), 0xf, 0xf, true)); \
        x[m] = __builtin_fmaf(arow[kk], xk_, x[m]);                                                             \
      }
      KDA_VSOLVE_STEP(0) KDA_VSOLVE_STEP(1) KDA_VSOLVE_STEP(2) KDA_VSOLVE_STEP(3) KDA_VSOLVE_STEP(4)
      KDA_VSOLVE_STEP(5) KDA_VSOLVE_STEP(6) KDA_VSOLVE_STEP(7) KDA_VSOLVE_STEP(8) KDA_VSOLVE_STEP(9)
      KDA_VSOLVE_STEP(10) KDA_VSOLVE_STEP(11) KDA_VSOLVE_STEP(12) KDA_VSOLVE_STEP(13) KDA_VSOLVE_STEP(14)
#undef KDA_VSOLVE_STEP
      *reinterpret_cast<uint2*>(&L.xh[lr][4 * g]) = make_uint2(pack2(h16(x[0]), h16(x[1])), pack2(h16(x[2]), h16(x[3])));
    }

    if constexpr (!FOLD) {
      // state slice to fp16 in LDS (this wave's own slice of sh, which only this wave reads), then
      // the whole next unit's slice into the registers it leaves
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t lo = pack2(h16(sv[i].x), h16(sv[i].y)), hi = pack2(h16(sv[i].z), h16(sv[i].w));
        *reinterpret_cast<uint2*>(&L.sh[wave][8 * i + (lane >> 3)][4 * (lane & 7)]) = make_uint2(lo, hi);
      }
      prefetch_state(srs, 0, 16);
    }
    // ---- Kt S0 (tokens x values) and (Qt S0)^T (values x tokens) on this wave's 32 columns
    f32x4 KS[2], QT[2];
    {
      const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
      KS[0] = KS[1] = QT[0] = QT[1] = z4;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 kr = perm_h(&L.kt[lr][32 * s], g);
        const f16x8 qr = perm_h(&L.qt[lr][32 * s], g);
#pragma unroll
        for (int nv = 0; nv < 2; ++nv) {
          // S0 rows {32s+4g+r} then {32s+16+4g+r}, column 16nv+lr of the slice, via the transposing read
          const uint16_t* p = &L.sh[wave][32 * s + 4 * g + (lr >> 2)][16 * nv + 4 * (lr & 3)];
          const f16x8 sf = as_f16x8(lds_tr(p), lds_tr(p + 16 * 32));
          KS[nv] = mfma_h(kr, sf, KS[nv]);
          QT[nv] = mfma_h(sf, qr, QT[nv]);
        }
      }
    }
    if constexpr (FOLD) prefetch_state(srs, kPiece2, 16);
    __syncthreads();  // X and P are complete

    // ---- R = diag(beta)(V - Kt S0), W = X R, O^T = scale (QT + W^T P^T)
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        A.o + row0 * D, 0, (ok && tn > 0) ? (int)((((uint32_t)tn - 1) * H + 1) * D * 4) : 0, kBufWord3);
    const f16x4 xa = __builtin_bit_cast(f16x4, lds8(&L.xh[lr][4 * g]));
    const f16x4 pa = __builtin_bit_cast(f16x4, lds8(&L.ph[lr][4 * g]));
    const float4 b4 = *reinterpret_cast<const float4*>(&L.beta[4 * g]);
    const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
    float mone = -1.0f;
    asm volatile("" : "+v"(mone));
#pragma unroll
    for (int nv = 0; nv < 2; ++nv) {
      const int col = 32 * wave + 16 * nv + lr;
      f32x4 R;
#pragma unroll
      for (int r = 0; r < 4; ++r) R[r] = bv[r] * (bf2f(L.v[4 * g + r][col]) - KS[nv][r]);
      const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
      f16x4 hi, lo;
      split_h4(R, hi, lo, mone);
      const f32x4 W = mfma_h16(xa, lo, mfma_h16(xa, hi, z4));
      split_h4(W, hi, lo, mone);
      const f32x4 O = mfma_h16(lo, pa, mfma_h16(hi, pa, QT[nv]));
      // lane (g, lr) holds O[t = lr][32w + 16nv + 4g + r]; rows t >= T fall outside the buffer
      // range and are dropped by the hardware
      const f32x4 os = {A.scale * O[0], A.scale * O[1], A.scale * O[2], A.scale * O[3]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, os), orsrc,
                                             (int)(((uint32_t)lr * H * D + 32 * wave + 16 * nv + 4 * g) * 4), 0, kStream);
    }
  }
}

bool verify_chunk_eligible(const VerifyArgs& a, bool f32_inputs) {
  return !f32_inputs && a.n_tok >= 1 && a.n_tok <= VT && a.commit_len == nullptr && a.fold_len == nullptr;
}

hipError_t launch_fold_verify(const VerifyArgs& a, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const long units = (long)a.batch * a.n_heads;
  const long slots = 2L * prefill_max_grid(dev);  // two resident workgroups per CU
  const dim3 grid((unsigned)(units < slots ? units : slots)), block(256);
  hipLaunchKernelGGL((verify_chunk_kernel<true, 8, true, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_verify_chunk(const VerifyArgs& a, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const long units = (long)a.batch * a.n_heads;
  const long per_cu = a.n_tok <= 8 ? 2 : 1;  // resident workgroups per CU (LDS-bound)
  const long slots = per_cu * prefill_max_grid(dev);
  const dim3 grid((unsigned)(units < slots ? units : slots)), block(256);
  const bool ring = a.ring_k != nullptr;
  if (a.cu_tok) {
    if (a.n_tok <= 8) {
      if (ring) hipLaunchKernelGGL((verify_chunk_kernel<true, 8, false, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((verify_chunk_kernel<false, 8, false, true>), grid, block, 0, stream, a);
    } else {
      if (ring) hipLaunchKernelGGL((verify_chunk_kernel<true, 16, false, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((verify_chunk_kernel<false, 16, false, true>), grid, block, 0, stream, a);
    }
  } else if (a.n_tok <= 8) {
    if (ring) hipLaunchKernelGGL((verify_chunk_kernel<true, 8, false, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((verify_chunk_kernel<false, 8, false, false>), grid, block, 0, stream, a);
  } else {
    if (ring) hipLaunchKernelGGL((verify_chunk_kernel<true, 16, false, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((verify_chunk_kernel<false, 16, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace kda
