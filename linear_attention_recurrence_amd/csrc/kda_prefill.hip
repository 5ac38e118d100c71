// kda_prefill.hip -- fused chunked prefill of the KDA recurrence on gfx950.
//
// Sources: Kimi K3 B200 deployment notes (zdszero.github.io), FlashKDA items
// of the optimisation timeline -- one kernel fuses a chunk's intra-chunk
// compute with the state update and keeps intermediates on chip; an fp32
// [128,128] state per (sequence, head); a persistent launch; longest-first
// (LPT) order of variable-length sequences; a host-built split plan reused by
// every layer. "SGLang and Miles Add Day-0 Support for Kimi K3" (LMSYS
// blog), section "Three state moves on the forward stream": snapshots at
// chunk boundaries into a ping-pong extra buffer.
//
// Algebra (the chunked form of the token recurrence; C = 32 tokens, chunk
// start state S0, G_t = sum_{tau<=t} gk_tau inside the chunk):
//   A[i][j] = beta_i sum_c Rk_ic Ck_jc     (j < i)   Rk = k e^{G - G_15}, Ck = k e^{G_15 - G}
//   P[t][i] =        sum_c Rq_tc Ck_ic     (i <= t)  Rq = q e^{G - G_15}
//   X = (I + A)^-1,   R = diag(beta) (V - Kt S0),   W = X R       Kt = k e^G
//   O = scale (Qt S0 + P W)                                       Qt = q e^G
//   S_end = e^{G_31} S0 + K'^T W                                  K' = k e^{G_31 - G}
// The intra-chunk factors are anchored at token 15 so each spans at most 16
// tokens of decay; every factor is a product of a = exp(gk) over such a
// span or its reciprocal, which stays in fp32/bf16 range when gk >= -5 (the
// documented precondition of this path). The factors of Kt, Qt, K' are <= 1.
//
// Precision (chosen by measuring each operand's rounding against the fp64
// oracle): the intra-chunk factors Rq and Ck enter their MFMAs as bf16 hi + lo
// pairs (Rk single), because their range needs bf16; every product that
// touches the state uses fp16 operands (11-bit significand), with R and W as
// fp16 hi + lo pairs. All accumulation is fp32 and the state stays fp32.
//
// Work decomposition: one 256-thread workgroup (4 waves) per (sequence, head)
// item, persistent, pulling items from a longest-first list with an atomic
// counter. Wave w owns value columns [32w, 32w+32); its 128x32 slice of the
// fp32 state lives in MFMA accumulator registers for the whole sequence and
// is fed back as the B operand of the next products by permuting the
// reduction index identically in both operands. Raw inputs of the next chunk
// stream into LDS with direct global->LDS loads while the current chunk
// computes; operands that a product needs transposed are read with the
// transposing LDS load (ds_read_b64_tr_b16) instead of being stored twice.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int C = 32;     // chunk length
constexpr int TM = 136;   // token-major row stride (16-bit elements; 128 + 8 pad)
constexpr int SQ = 40;    // 32x32 16-bit matrices
constexpr int ATS = 36;   // 32x32 fp32 matrices

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct PrefillLds {
  // operands of the current chunk, token-major [t][c]
  uint16_t qt[C][TM];                  // fp16  q e^G
  uint16_t kt[C][TM];                  // fp16  k e^G
  uint16_t kp[C][TM];                  // fp16  k e^{G_31 - G}
  uint16_t vt[C][TM];                  // bf16  v (copy out of the staging area)
  float part[4][6][16][20];            // per-wave partial A and P tiles over 32 channels, [col][row] (padded)
  float at[C][ATS];                    // A transposed: at[j][i] = A[i][j]
  float xf[C][ATS];                    // diagonal blocks of X, fp32
  uint16_t xb[C][SQ];                  // fp16 X, rows t, columns j
  uint16_t pm[C][SQ];                  // fp16 P, rows t, columns i
  float beta[C];
  float dlast[D];                      // e^{G_31} per key channel
  float so[C][D];                      // output tile of the previous chunk, flushed as whole rows
  int item;
};

__device__ __forceinline__ uint2 lds8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint4 lds16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// 16 (or 4) bytes per lane from global memory into LDS at lds_base + size * lane
// (lds_base wave-uniform). Written as inline assembly on purpose: the compiler
// would otherwise make every later LDS read wait for these asynchronous
// writes, which turns the one-chunk-ahead prefetch into a synchronous load.
// The kernel orders them itself: s_waitcnt vmcnt(0) plus a barrier before the
// staging area is read. M0 is used by nothing else in this kernel.
__device__ __forceinline__ void g2l(const void* src, void* lds_base, int bytes) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_base);
  if (bytes == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(m0), "v"(src) : "memory");
}

// transposing read: within each 16-lane group, lane j gets element r from the
// 4-element row chunk that lane 4r + j/4 points at, position j % 4
__device__ __forceinline__ uint2 lds_tr(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

__device__ __forceinline__ f32x4 mfma_h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 as_f16x8(uint2 a, uint2 b) {
  return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// permuted A operand of a 32-wide reduction step: row elements {4g..4g+3} then {16+4g..16+4g+3}
__device__ __forceinline__ f16x8 perm_h(const uint16_t* row, int g) { return as_f16x8(lds8(row + 4 * g), lds8(row + 16 + 4 * g)); }

// B operand from two accumulator tiles (rows 4g+r of tile 0, then of tile 1): fp16, and hi/lo
__device__ __forceinline__ f16x8 to_h8(const f32x4& a, const f32x4& b) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = (_Float16)a[i]; r[4 + i] = (_Float16)b[i]; }
  return r;
}
__device__ __forceinline__ void split_h8(const f32x4& a, const f32x4& b, f16x8& hi, f16x8& lo) {
  hi = to_h8(a, b);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = (_Float16)(a[i] - (float)hi[i]);
    lo[4 + i] = (_Float16)(b[i] - (float)hi[4 + i]);
  }
}

#define KDA_ROW_SHR(v, s) __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(v), 0x110 + (s), 0xf, 0xf, false))
#define KDA_ROW_BCAST15(v) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x15F, 0xf, 0xf, false))

// inclusive prefix product over the 16 lanes of a DPP row (lane order = token order)
__device__ __forceinline__ float row_scan_mul(float v) {
  v = v * KDA_ROW_SHR(v, 1);
  v = v * KDA_ROW_SHR(v, 2);
  v = v * KDA_ROW_SHR(v, 4);
  v = v * KDA_ROW_SHR(v, 8);
  return v;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = bf2f(w[i] & 0xffffu); f[2 * i + 1] = bf2f(w[i] >> 16); }
}
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) { return pack2(f2bf(a), f2bf(b)); }
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  return pack2(__builtin_bit_cast(uint16_t, (_Float16)a), __builtin_bit_cast(uint16_t, (_Float16)b));
}
// 8 products written as one 16-byte row chunk: bf16, bf16 hi/lo, or fp16
__device__ __forceinline__ void put_bf16(uint16_t* dst, const float (&x)[8]) {
  *reinterpret_cast<uint4*>(dst) = make_uint4(pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]), pk_bf16(x[4], x[5]), pk_bf16(x[6], x[7]));
}
__device__ __forceinline__ void put_bf16_split(uint16_t* hi, uint16_t* lo, const float (&x)[8]) {
  uint16_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split_bf16(x[i], h[i], l[i]);
  *reinterpret_cast<uint4*>(hi) = make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
  *reinterpret_cast<uint4*>(lo) = make_uint4(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
}
__device__ __forceinline__ void put_f16(uint16_t* dst, const float (&x)[8]) {
  *reinterpret_cast<uint4*>(dst) = make_uint4(pk_f16(x[0], x[1]), pk_f16(x[2], x[3]), pk_f16(x[4], x[5]), pk_f16(x[6], x[7]));
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_kernel(PrefillArgs A) {
  __shared__ PrefillLds L;
  // raw inputs of the next chunk, written by direct global->LDS loads
  __shared__ uint16_t Sq[C][D], Sk[C][D], Sv[C][D];
  __shared__ float Sg[C][D];
  __shared__ float Sbeta[C];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, lr = lane & 15;  // MFMA lane group and lane row/column
  const int co = 4 * wave + g;              // prep: channel octet 8co..8co+7
  const int tl = lr;                        // prep: token tl of block 0 and 16+tl of block 1
  const int H = A.n_heads;
  const int wu = __builtin_amdgcn_readfirstlane(wave);

  // constant zero blocks: A, P and X are lower triangular in 16-blocks
  for (int e = tid; e < 16 * 16; e += 256) {
    const int i = e >> 4, j = 16 + (e & 15);
    L.at[j][i] = 0.f;
    L.pm[i][j] = 0;
    L.xb[i][j] = 0;
  }

  for (;;) {
    __syncthreads();
    if (tid == 0) L.item = atomicAdd(&A.ws->counter, 1);
    __syncthreads();
    const int it = L.item;
    if (it < 0 || it >= A.n_items) break;  // also ends a launch on a stale counter
    const int4 wi = A.items[it];
    const int n = wi.x, h = wi.y;
    const int64_t tok0 = wi.z;
    const int len = wi.w;
    if (n < 0 || n >= A.n_seq || h < 0 || h >= H || tok0 < 0 || len < 0 || tok0 + len > A.total_tokens) continue;
    const size_t unit = (size_t)n * H + h;

    // state slice of this wave in accumulator layout: S[mc][nv] holds rows 16mc+4g+r, column 32w+16nv+lr
    f32x4 S[8][2];
    if (A.state_in) {
      const float* src = A.state_in + unit * D * D;
#pragma unroll
      for (int mc = 0; mc < 8; ++mc)
#pragma unroll
        for (int nv = 0; nv < 2; ++nv)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[mc][nv][r] = src[(size_t)(16 * mc + 4 * g + r) * D + 32 * wave + 16 * nv + lr];
    } else {
#pragma unroll
      for (int mc = 0; mc < 8; ++mc)
#pragma unroll
        for (int nv = 0; nv < 2; ++nv) S[mc][nv] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Raw inputs of a chunk are copied into LDS with direct global->LDS loads
    // issued one chunk ahead; rows past the sequence end re-read its last
    // token (always in bounds) and are masked in the prep.
    const int nch = (len + C - 1) / C;
    // Staging rows are stored with their 16-byte chunks permuted (physical
    // chunk = logical chunk ^ (row & 15)) so the prep's column reads across 16
    // rows hit 16 different LDS banks; each lane fetches the chunk that lands
    // in its fixed LDS slot.
    auto issue = [&](int ch) {
      const int nc = min(C, len - C * ch);
      const int64_t trow0 = tok0 + C * ch;
#pragma unroll
      for (int r = 0; r < 2; ++r) {  // q, k, v: 256-byte rows (16 chunks), 4 rows per wave
        const int prow = 16 * r + 4 * wu + (lane >> 4);
        const int row = min(prow, nc - 1);
        const size_t e = ((size_t)(trow0 + row) * H + h) * D + 8 * ((lane & 15) ^ (prow & 15));
        g2l(A.q + e, &Sq[16 * r + 4 * wu][0], 16);
        g2l(A.k + e, &Sk[16 * r + 4 * wu][0], 16);
        g2l(A.v + e, &Sv[16 * r + 4 * wu][0], 16);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // gk: 512-byte rows (32 chunks), 2 rows per wave
        const int prow = 8 * r + 2 * wu + (lane >> 5);
        const int row = min(prow, nc - 1);
        const size_t e = ((size_t)(trow0 + row) * H + h) * D + 4 * ((lane & 31) ^ (prow & 15));
        g2l(A.gk + e, &Sg[8 * r + 2 * wu][0], 16);
      }
      if (wu == 0 && lane < C) g2l(A.beta + (size_t)(trow0 + min(lane, nc - 1)) * H + h, &Sbeta[0], 4);
    };
    // whole-row stores of a staged output tile (8 threads x 64 bytes per token row)
    auto flush = [&](int ch) {
      const int nc = min(C, len - C * ch);
      const int row = tid >> 3, c0 = 16 * (tid & 7);
      if (row < nc) {
        float* dst = A.o + ((size_t)(tok0 + C * ch + row) * H + h) * D + c0;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(dst + 4 * q4) = *reinterpret_cast<const float4*>(&L.so[row][c0 + 4 * q4]);
      }
    };
    if (nch > 0) issue(0);

    for (int ch = 0; ch < nch; ++ch) {
      const int nc = min(C, len - C * ch);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's staging loads (and older stores) are complete
      __syncthreads();
      if (ch > 0) flush(ch - 1);

      // ---------------- prep: decay factors and operand matrices ----------------
      {
        const int c8 = 8 * co;
        const bool ok0 = tl < nc, ok1 = 16 + tl < nc;
        float a0[8], a1[8];
        {
          // logical gk chunks 2co and 2co+1 of rows tl and 16+tl, at their permuted positions
          const float4 x0 = *reinterpret_cast<const float4*>(&Sg[tl][4 * ((2 * co) ^ tl)]);
          const float4 x1 = *reinterpret_cast<const float4*>(&Sg[tl][4 * ((2 * co + 1) ^ tl)]);
          const float4 y0 = *reinterpret_cast<const float4*>(&Sg[16 + tl][4 * ((2 * co) ^ tl)]);
          const float4 y1 = *reinterpret_cast<const float4*>(&Sg[16 + tl][4 * ((2 * co + 1) ^ tl)]);
          const float gx[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          const float gy[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) { a0[i] = ok0 ? __expf(gx[i]) : 1.f; a1[i] = ok1 ? __expf(gy[i]) : 1.f; }
        }
        const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
        const int sc = 8 * (co ^ tl);  // permuted position of logical chunk co (rows tl and 16+tl share row & 15)
        const uint4 k0u = ok0 ? lds16(&Sk[tl][sc]) : zero4, k1u = ok1 ? lds16(&Sk[16 + tl][sc]) : zero4;
        const uint4 q0u = ok0 ? lds16(&Sq[tl][sc]) : zero4, q1u = ok1 ? lds16(&Sq[16 + tl][sc]) : zero4;
        *reinterpret_cast<uint4*>(&L.vt[tl][c8]) = ok0 ? lds16(&Sv[tl][sc]) : zero4;
        *reinterpret_cast<uint4*>(&L.vt[16 + tl][c8]) = ok1 ? lds16(&Sv[16 + tl][sc]) : zero4;
        if (tid < C) L.beta[tid] = tid < nc ? Sbeta[tid] : 0.f;
        float k0[8], k1[8], q0[8], q1[8];
        unpack_bf16x8(k0u, k0); unpack_bf16x8(k1u, k1);
        unpack_bf16x8(q0u, q0); unpack_bf16x8(q1u, q1);
        float xr0[8], xr1[8], yc0[8], yc1[8], e0[8], e1[8], f0[8], f1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = row_scan_mul(a0[i]), p1 = row_scan_mul(a1[i]);  // e^{G_t - G_-1}, e^{G_t - G_15}
          const float T0 = KDA_ROW_BCAST15(p0), T1 = KDA_ROW_BCAST15(p1);   // block totals
          const float r0 = __builtin_amdgcn_rcpf(p0), r1 = __builtin_amdgcn_rcpf(p1);
          xr0[i] = p0 * __builtin_amdgcn_rcpf(T0);  // e^{G_t - G_15}, block 0
          xr1[i] = p1;
          yc0[i] = T0 * r0;                         // e^{G_15 - G_t}, block 0
          yc1[i] = r1;
          e0[i] = p0;                               // e^{G_t}
          e1[i] = T0 * p1;
          f0[i] = yc0[i] * T1;                      // e^{G_31 - G_t}
          f1[i] = T1 * r1;
          if (tl == 0) L.dlast[c8 + i] = T0 * T1;
        }
        // fp16 operands of the state products, token-major rows tl and 16+tl
        float x[8];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int t = 16 * b + tl;
          const float(&kk)[8] = b ? k1 : k0;
          const float(&qq)[8] = b ? q1 : q0;
          const float(&ee)[8] = b ? e1 : e0;
          const float(&ff)[8] = b ? f1 : f0;
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = qq[i] * ee[i];
          put_f16(&L.qt[t][c8], x);
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = kk[i] * ee[i];
          put_f16(&L.kt[t][c8], x);
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = kk[i] * ff[i];
          put_f16(&L.kp[t][c8], x);
        }
        // A and P over this wave's 32 channels, straight from registers: lane (g, lr) holds
        // channels 32w+8g..+7 of tokens lr (block 0) and 16+lr (block 1), which is the
        // A-operand fragment of row lr and the B-operand fragment of column lr
        bf16x8 rk0, rk1, rq0h, rq0l, rq1h, rq1l, ck0h, ck0l, ck1h, ck1l;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          rk0[i] = (__bf16)(k0[i] * xr0[i]);
          rk1[i] = (__bf16)(k1[i] * xr1[i]);
          float v = q0[i] * xr0[i]; rq0h[i] = (__bf16)v; rq0l[i] = (__bf16)(v - (float)rq0h[i]);
          v = q1[i] * xr1[i];       rq1h[i] = (__bf16)v; rq1l[i] = (__bf16)(v - (float)rq1h[i]);
          v = k0[i] * yc0[i];       ck0h[i] = (__bf16)v; ck0l[i] = (__bf16)(v - (float)ck0h[i]);
          v = k1[i] * yc1[i];       ck1h[i] = (__bf16)v; ck1l[i] = (__bf16)(v - (float)ck1h[i]);
        }
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 acc[6];
        acc[0] = mfma16(rk0, ck0l, mfma16(rk0, ck0h, z4));                          // A 00
        acc[1] = mfma16(rk1, ck1l, mfma16(rk1, ck1h, z4));                          // A 11
        acc[2] = mfma16(rk1, ck0l, mfma16(rk1, ck0h, z4));                          // A 10
        acc[3] = mfma16(rq0l, ck0h, mfma16(rq0h, ck0l, mfma16(rq0h, ck0h, z4)));   // P 00
        acc[4] = mfma16(rq1l, ck1h, mfma16(rq1h, ck1l, mfma16(rq1h, ck1h, z4)));   // P 11
        acc[5] = mfma16(rq1l, ck0h, mfma16(rq1h, ck0l, mfma16(rq1h, ck0h, z4)));   // P 10
#pragma unroll
        for (int tl6 = 0; tl6 < 6; ++tl6)
          *reinterpret_cast<f32x4*>(&L.part[wave][tl6][lr][4 * g]) = acc[tl6];
      }
      __syncthreads();
      // the staging area is consumed: next chunk's raw inputs stream in while this chunk computes
      if (ch + 1 < nch) issue(ch + 1);

      // reduce the four channel slices of A and P; mask, scale A rows by beta
      if (tid < 192) {
        const int tile = tid >> 5, j = (tid >> 1) & 15, i0 = 8 * (tid & 1);
        const int I = (tile % 3) == 0 ? 0 : 1, J = (tile % 3) == 1 ? 1 : 0;
        float sum[8];
#pragma unroll
        for (int q8 = 0; q8 < 2; ++q8) {
          f32x4 s4 = *reinterpret_cast<const f32x4*>(&L.part[0][tile][j][i0 + 4 * q8]);
#pragma unroll
          for (int w = 1; w < 4; ++w) {
            const f32x4 p4 = *reinterpret_cast<const f32x4*>(&L.part[w][tile][j][i0 + 4 * q8]);
            s4[0] += p4[0]; s4[1] += p4[1]; s4[2] += p4[2]; s4[3] += p4[3];
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) sum[4 * q8 + r] = s4[r];
        }
        const int jg = 16 * J + j;
        if (tile < 3) {
          float av[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int ig = 16 * I + i0 + r;
            av[r] = (jg < ig) ? sum[r] * L.beta[ig] : 0.f;
          }
          *reinterpret_cast<float4*>(&L.at[jg][16 * I + i0]) = make_float4(av[0], av[1], av[2], av[3]);
          *reinterpret_cast<float4*>(&L.at[jg][16 * I + i0 + 4]) = make_float4(av[4], av[5], av[6], av[7]);
        } else {
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int ig = 16 * I + i0 + r;
            L.pm[ig][jg] = (jg <= ig) ? __builtin_bit_cast(uint16_t, (_Float16)sum[r]) : (uint16_t)0;
          }
        }
      }
      __syncthreads();  // A (transposed, fp32) and P (fp16) are complete

      // ---------------- X = (I + A)^-1 (wave 0) ----------------
      if (wave == 0) {
        if (lane < 32) {
          // diagonal blocks by forward substitution, one column per lane
          const int b = lane >> 4, jl = lane & 15;
          float xv[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) xv[i] = (i == jl) ? 1.f : 0.f;
#pragma unroll
          for (int kk = 0; kk < 15; ++kk) {
            const float* col = &L.at[16 * b + kk][16 * b];  // A[16b+i][16b+kk], i = 0..15
            float av[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const float4 t4 = *reinterpret_cast<const float4*>(col + 4 * q4);
              av[4 * q4] = t4.x; av[4 * q4 + 1] = t4.y; av[4 * q4 + 2] = t4.z; av[4 * q4 + 3] = t4.w;
            }
            const float xk = xv[kk];
#pragma unroll
            for (int i = kk + 1; i < 16; ++i) xv[i] = __builtin_fmaf(-av[i], xk, xv[i]);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            L.xf[16 * b + i][16 * b + jl] = xv[i];
            L.xb[16 * b + i][16 * b + jl] = __builtin_bit_cast(uint16_t, (_Float16)xv[i]);
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        // X10 = -X11 (A10 X00) with fp32 MFMAs; the reduction index of step s in lane group g is 4g+s
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) y = mfma_f32(L.at[4 * g + s][16 + lr], L.xf[4 * g + s][lr], y);
        f32x4 x10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) x10 = mfma_f32(L.xf[16 + lr][16 + 4 * g + s], y[s], x10);
#pragma unroll
        for (int r = 0; r < 4; ++r) L.xb[16 + 4 * g + r][lr] = __builtin_bit_cast(uint16_t, (_Float16)(-x10[r]));
      }

      // ---------------- Kt S0 and Qt S0 (independent of X) ----------------
      f32x4 KS[2][2], QS[2][2];
      {
        f16x8 Sh[4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int nv = 0; nv < 2; ++nv) Sh[s][nv] = to_h8(S[2 * s][nv], S[2 * s + 1][nv]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int nv = 0; nv < 2; ++nv) { KS[mt][nv] = f32x4{0.f, 0.f, 0.f, 0.f}; QS[mt][nv] = f32x4{0.f, 0.f, 0.f, 0.f}; }
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int m = 16 * mt + lr;
            const f16x8 kr = perm_h(&L.kt[m][32 * s], g);
            const f16x8 qr = perm_h(&L.qt[m][32 * s], g);
#pragma unroll
            for (int nv = 0; nv < 2; ++nv) {
              KS[mt][nv] = mfma_h(kr, Sh[s][nv], KS[mt][nv]);
              QS[mt][nv] = mfma_h(qr, Sh[s][nv], QS[mt][nv]);
            }
          }
        }
      }
      __syncthreads();  // X is complete

      // ---------------- R = diag(beta)(V - Kt S0), W = X R ----------------
      f32x4 W[2][2];
      {
        f16x8 Rh[2], Rl[2];
#pragma unroll
        for (int nv = 0; nv < 2; ++nv) {
          f32x4 R[2];
          const int c0 = 32 * wave + 16 * nv;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            // V[16mt+4g+r][c0+lr] through the transposing read
            const uint2 vv = lds_tr(&L.vt[16 * mt + 4 * g + (lr >> 2)][c0 + 4 * (lr & 3)]);
            const float4 b4 = *reinterpret_cast<const float4*>(&L.beta[16 * mt + 4 * g]);
            R[mt][0] = b4.x * (bf2f(vv.x & 0xffffu) - KS[mt][nv][0]);
            R[mt][1] = b4.y * (bf2f(vv.x >> 16) - KS[mt][nv][1]);
            R[mt][2] = b4.z * (bf2f(vv.y & 0xffffu) - KS[mt][nv][2]);
            R[mt][3] = b4.w * (bf2f(vv.y >> 16) - KS[mt][nv][3]);
          }
          split_h8(R[0], R[1], Rh[nv], Rl[nv]);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const f16x8 xa = perm_h(&L.xb[16 * mt + lr][0], g);
#pragma unroll
          for (int nv = 0; nv < 2; ++nv) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma_h(xa, Rh[nv], acc);
            acc = mfma_h(xa, Rl[nv], acc);
            W[mt][nv] = acc;
          }
        }
      }
      f16x8 Wh[2], Wl[2];
#pragma unroll
      for (int nv = 0; nv < 2; ++nv) split_h8(W[0][nv], W[1][nv], Wh[nv], Wl[nv]);

      // ---------------- O = scale (Qt S0 + P W) into the output staging tile ----------------
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f16x8 pa = perm_h(&L.pm[16 * mt + lr][0], g);
#pragma unroll
        for (int nv = 0; nv < 2; ++nv) {
          f32x4 acc = QS[mt][nv];
          acc = mfma_h(pa, Wh[nv], acc);
          acc = mfma_h(pa, Wl[nv], acc);
          const int v = 32 * wave + 16 * nv + lr;
#pragma unroll
          for (int r = 0; r < 4; ++r) L.so[16 * mt + 4 * g + r][v] = A.scale * acc[r];
        }
      }

      // ---------------- S = e^{G_31} S0 + K'^T W ----------------
#pragma unroll
      for (int mc = 0; mc < 8; ++mc) {
        const float4 d4 = *reinterpret_cast<const float4*>(&L.dlast[16 * mc + 4 * g]);
        // K'^T rows 16mc+lr, reduction positions t = 4g+r and 16+4g+r, via the transposing read
        const uint16_t* base = &L.kp[4 * g + (lr >> 2)][16 * mc + 4 * (lr & 3)];
        const f16x8 ka = as_f16x8(lds_tr(base), lds_tr(base + 16 * TM));
#pragma unroll
        for (int nv = 0; nv < 2; ++nv) {
          f32x4 acc = S[mc][nv];
          acc[0] *= d4.x; acc[1] *= d4.y; acc[2] *= d4.z; acc[3] *= d4.w;
          acc = mfma_h(ka, Wh[nv], acc);
          acc = mfma_h(ka, Wl[nv], acc);
          S[mc][nv] = acc;
        }
      }

      // ---------------- snapshot at chunk ends p with p % interval == 0 ----------------
      const int p = C * ch + nc;
      if (A.snap_interval > 0 && p % A.snap_interval == 0) {
        const int m = p / A.snap_interval;
        float* dst = A.snap + (((size_t)n * A.snap_slots + (m - 1) % A.snap_slots) * H + h) * D * D;
#pragma unroll
        for (int mc = 0; mc < 8; ++mc)
#pragma unroll
          for (int nv = 0; nv < 2; ++nv)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(size_t)(16 * mc + 4 * g + r) * D + 32 * wave + 16 * nv + lr] = S[mc][nv][r];
      }
    }
    __syncthreads();
    if (nch > 0) flush(nch - 1);

    float* dst = A.state_out + unit * D * D;
#pragma unroll
    for (int mc = 0; mc < 8; ++mc)
#pragma unroll
      for (int nv = 0; nv < 2; ++nv)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(size_t)(16 * mc + 4 * g + r) * D + 32 * wave + 16 * nv + lr] = S[mc][nv][r];
    if (A.snap_count && h == 0 && tid == 0) A.snap_count[n] = A.snap_interval > 0 ? len / A.snap_interval : 0;
  }

  // the last workgroup out resets the counters, so a later launch with the
  // same resident work list starts from zero
  if (tid == 0) {
    __threadfence();
    const int d = atomicAdd(&A.ws->done, 1);
    if (d == (int)gridDim.x - 1) {
      atomicExch(&A.ws->counter, 0);
      atomicExch(&A.ws->done, 0);
    }
  }
}

int prefill_max_grid(int device) {
  static int cus[64] = {0};
  if (device < 0 || device >= 64) return 256;
  if (cus[device] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0) n = 256;
    cus[device] = n;
  }
  return cus[device];  // one 256-thread workgroup per CU (LDS-bound)
}

hipError_t launch_prefill(const PrefillArgs& a, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
