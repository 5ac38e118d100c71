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
//   A[i][j] = beta_i sum_c Kt_ic Ck_jc     (j < i)   Kt = k e^G, Ck = k e^{-G}
//   P[t][i] =        sum_c Qt_tc Ck_ic     (i <= t)  Qt = q e^G
//   X = (I + A)^-1,   R = diag(beta) (V - Kt S0),   W = X R
//   O = scale (Qt S0 + P W)
//   S_end = e^{G_31} S0 + K'^T W                                  K' = k e^{G_31 - G}
// Kt and Qt serve both as the chain's fp16 operands and, rounded to bf16, as
// the row factors of A and P. The column factor e^{-G} grows with the decay
// summed over the chunk; every factor stays in fp32/bf16 range, with its bf16
// low part normal, while that sum is at most 60 per key channel. Beyond it
// (or for gk = -inf) the item is computed again in a form with the exact path
// below (see kMinChunkDecay).
//
// Precision (chosen by measuring each operand's rounding against the fp64
// oracle): the intra-chunk factors Rq and Ck enter their MFMAs as bf16 hi + lo
// pairs (Rk single), because their range needs bf16; every product that
// touches the state uses fp16 operands (11-bit significand), with R and W as
// fp16 hi + lo pairs. All accumulation is fp32 and the state stays fp32.
//
// Work decomposition: one 512-thread workgroup per CU, persistent, pulling
// (sequence, head, value block) items from a longest-first list with an atomic
// counter. A value block is all 128 value columns of the state, or one half
// of them when the plan splits chains (the columns evolve independently given
// the key side, which each half recomputes).
// Inside an item the workgroup is a two-stage pipeline over chunks, one
// period per chunk, each period cut in two phases by workgroup barriers:
//   consumer waves 0-3 run the serial state chain of chunk c. Wave w owns
//     value columns [32w, 32w+32) (in a half-chain [64vb + 16w, +16)); its
//     128x32 (128x16) slice of the fp32 state lives
//     in MFMA accumulator registers for the whole sequence and is fed back as
//     the B operand of the next products by permuting the reduction index
//     identically in both operands. Phase 1: Kt S0, Qt S0, R, W = X R and
//     O = Qt S0 + P W (stored straight from the accumulators), then the
//     state update and the snapshot (they read only this chunk's rows,
//     written one period earlier); phase 2: the sums below.
//   producer waves 4-7 prepare chunk c+1. Phase 1: raw q, k, gk, beta
//     (prefetched into registers two periods ahead, the set's gk already
//     turned into prefix sums) become decay factors, per-wave partial A and
//     P tiles and the fp16 operand rows of the chain, and the q and k loads
//     of chunk c+3 go out. Phase 2: the gk and beta loads of chunk c+3, the
//     next set's prefix sums, raw v of chunk c+2 from global memory straight
//     into LDS (global_load_lds) for the chain, and the operand rows to LDS;
//     meanwhile the consumer waves turn the partials into the next chunk's X
//     (waves 0 and 3 invert one diagonal block of I + A each), P (wave 1) and
//     -A10 (wave 2).
// Everything the two stages exchange is double-buffered by chunk parity, so
// a period needs just its two barriers. Operands that a product needs
// transposed are read with the transposing LDS load (ds_read_b64_tr_b16)
// instead of being stored twice.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_norm.h"

namespace kda {

typedef __attribute__((ext_vector_type(2))) unsigned u32x2v;

constexpr int C = 32;      // chunk length
constexpr int TM = 152;    // token-major row stride (16-bit elements; 128 + 24 pad: rows 12 banks apart)
constexpr int SQ = 40;     // 32x32 16-bit matrices
constexpr int ATS = 36;    // 32x32 fp32 matrices
constexpr int NT = 512;    // threads per workgroup: 4 consumer + 4 producer waves

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct alignas(16) PrefillLds {
  // chain operands, double-buffered by chunk parity; token-major [t][c]
  uint16_t qt[2][C][TM];               // fp16  q e^G
  uint16_t kt[2][C][TM];               // fp16  k e^G
  uint16_t kp[2][C][TM];               // fp16  k e^{G_31 - G}
  uint16_t vr[2][C][D];                // bf16  raw v, 16-byte chunks stored at chunk ^ (2 row & 15)
  uint16_t xb[2][C][SQ];               // fp16  diagonal 16-blocks of X = (I + A)^-1, rows t, columns j
  uint16_t an[2][16][SQ];              // fp16  -A[16 + i][j], the off-diagonal block of A
  uint16_t pm[2][C][SQ];               // fp16  P, rows t, columns i
  float beta[2][C];
  float dlast[2][D];                   // e^{G_31} per key channel
  // partial tiles (producers write, the chain sums) and the solve's scratch
  float part[4][6][16][20];            // per-wave partial A and P tiles over 32 channels, [col][row] (padded)
  float ar[C][ATS];                    // diagonal blocks of A, fp32, rows i
  int item;
  int redo;                            // set when a chunk of the item is beyond the factor form's range
  // the fused output norm (kda_chunk_prefill_gated): raw gate rows (stored like vr), per-token slice
  // sums of squares of o, and the norm weights
  uint16_t gr[2][C][D];
  float ssq[C][16];   // slice sums of squares of the chunk's o, [token][slice]
  float rs[C];        // 1 / rms of each token row
  float nw[D];
};

__device__ __forceinline__ uint2 lds8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane
// (lds_base wave-uniform). Written as inline assembly on purpose: the compiler
// would otherwise make every later LDS read wait for these asynchronous
// writes. The kernel orders them itself: before the barrier that ends a period
// the issuing wave waits until only that period's loads are in flight (vmcnt),
// so rows issued one period earlier have landed before the chain reads them in
// the next period. M0 is used by nothing else here.
__device__ __forceinline__ void g2l16(const void* src, void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory");
}

// transposing read: within each 16-lane group, lane j gets element r from the
// 4-element row chunk that lane 4r + j/4 points at, position j % 4
__device__ __forceinline__ uint2 lds_tr(const uint16_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

__device__ __forceinline__ f32x4 mfma_h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 16x16x16 fp16 MFMA: lane l holds A[l%16][4(l/16)+i], B[4(l/16)+i][l%16] (i < 4)
__device__ __forceinline__ f32x4 mfma_h16(const f16x4& a, const f16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
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
// fp16 hi + lo of two fp32 values: hi = f16(x), lo = f16(x - hi). The remainder x - hi is exact
// in fp32; it is formed by one fused multiply-add that takes the packed fp16 hi as its operand
// (the mixed-precision FMA), instead of converting hi back to fp32 and subtracting. The empty
// asm keeps the packed hi as the operand rather than a second scalar conversion of x.
__device__ __forceinline__ void split_pair(float x, float y, f16x2& hi, f16x2& lo, float mone) {
  hi = f16x2{(_Float16)x, (_Float16)y};
  asm("" : "+v"(hi));
  lo = f16x2{(_Float16)__builtin_fmaf((float)hi[0], mone, x), (_Float16)__builtin_fmaf((float)hi[1], mone, y)};
}
// -1.0f in a register: with a literal the compiler folds the FMA back into a subtraction
__device__ __forceinline__ float minus_one() {
  float m = -1.0f;
  asm volatile("" : "+v"(m));
  return m;
}
__device__ __forceinline__ void split_h4(const f32x4& a, f16x4& hi, f16x4& lo, float mone) {
  f16x2 h0, l0, h1, l1;
  split_pair(a[0], a[1], h0, l0, mone);
  split_pair(a[2], a[3], h1, l1, mone);
  hi = f16x4{h0[0], h0[1], h1[0], h1[1]};
  lo = f16x4{l0[0], l0[1], l1[0], l1[1]};
}
__device__ __forceinline__ void split_h8(const f32x4& a, const f32x4& b, f16x8& hi, f16x8& lo, float mone) {
  f16x4 ha, la, hb, lb;
  split_h4(a, ha, la, mone);
  split_h4(b, hb, lb, mone);
  hi = f16x8{ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
  lo = f16x8{la[0], la[1], la[2], la[3], lb[0], lb[1], lb[2], lb[3]};
}

// row_shr:s with bound_ctrl: lanes shifted in from outside the 16-lane DPP row read 0
#define KDA_ROW_SHR0(v, s) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x110 + (s), 0xf, 0xf, true))
#define KDA_ROW_BCAST15(v) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x15F, 0xf, 0xf, true))

// inclusive prefix sum over the 16 lanes of a DPP row (lane order = token order)
__device__ __forceinline__ float row_scan_add(float v) {
  v = v + KDA_ROW_SHR0(v, 1);
  v = v + KDA_ROW_SHR0(v, 2);
  v = v + KDA_ROW_SHR0(v, 4);
  v = v + KDA_ROW_SHR0(v, 8);
  return v;
}

// row_shl:s with bound_ctrl: lane t reads lane t + s of its DPP row, 0 past the row's end
#define KDA_ROW_SHL0(v, s) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x100 + (s), 0xf, 0xf, true))

// exclusive suffix sum over the 16 lanes of a DPP row: lane t gets the sum of lanes t+1 .. 15
__device__ __forceinline__ float row_suffix_excl(float v) {
  v = v + KDA_ROW_SHL0(v, 1);
  v = v + KDA_ROW_SHL0(v, 2);
  v = v + KDA_ROW_SHL0(v, 4);
  v = v + KDA_ROW_SHL0(v, 8);
  return KDA_ROW_SHL0(v, 1);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = bf2f(w[i] & 0xffffu); f[2 * i + 1] = bf2f(w[i] >> 16); }
}
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
}

// Raw inputs of one chunk as one producer lane needs them: channel octet
// 8co..8co+7 of tokens tl and 16+tl (rows past the sequence end re-read its
// last token, always in bounds; gk and beta are masked where they are used).
struct Raw {
  uint4 q0, q1, k0, k1;
  float4 g0a, g0b, g1a, g1b;
  float b0, b1;
};

// row0: (first token of the chunk) * H + h, wave-uniform. Per-lane offsets are 32-bit byte
// offsets from wave-uniform bases, so the loads take the scalar-base addressing form.
// Tokens past the chunk end re-read the last token (finite values; see stage1).
__device__ __forceinline__ void load_raw(Raw& r, const PrefillArgs& A, size_t row0, int nc, int co, int tl) {
  const uint32_t HD2 = (uint32_t)A.n_heads * (D * 2);  // bytes per token of a bf16 [T, H, D] tensor
  const uint32_t t0 = (uint32_t)min(tl, nc - 1), t1 = (uint32_t)min(16 + tl, nc - 1);
  const uint32_t b0 = t0 * HD2 + 16u * co, b1 = t1 * HD2 + 16u * co;
  const char* q = reinterpret_cast<const char*>(A.q + row0 * D);
  const char* k = reinterpret_cast<const char*>(A.k + row0 * D);
  const char* gk = reinterpret_cast<const char*>(A.gk + row0 * D);  // fp32: twice the bf16 offsets
  const char* beta = reinterpret_cast<const char*>(A.beta + row0);
  const uint32_t H4 = (uint32_t)A.n_heads * 4u;
  r.q0 = *reinterpret_cast<const uint4*>(q + b0);
  r.q1 = *reinterpret_cast<const uint4*>(q + b1);
  r.k0 = *reinterpret_cast<const uint4*>(k + b0);
  r.k1 = *reinterpret_cast<const uint4*>(k + b1);
  r.g0a = *reinterpret_cast<const float4*>(gk + 2u * b0);
  r.g0b = *reinterpret_cast<const float4*>(gk + 2u * b0 + 16u);
  r.g1a = *reinterpret_cast<const float4*>(gk + 2u * b1);
  r.g1b = *reinterpret_cast<const float4*>(gk + 2u * b1 + 16u);
  r.b0 = *reinterpret_cast<const float*>(beta + t0 * H4);
  r.b1 = *reinterpret_cast<const float*>(beta + t1 * H4);
}

// the two halves of load_raw: q and k (issued during phase 1, once the set's q and k are unpacked),
// then gk and beta (issued in phase 2)
__device__ __forceinline__ void load_raw_qk(Raw& r, const PrefillArgs& A, size_t row0, int nc, int co, int tl) {
  const uint32_t HD2 = (uint32_t)A.n_heads * (D * 2);
  const uint32_t t0 = (uint32_t)min(tl, nc - 1), t1 = (uint32_t)min(16 + tl, nc - 1);
  const uint32_t b0 = t0 * HD2 + 16u * co, b1 = t1 * HD2 + 16u * co;
  const char* q = reinterpret_cast<const char*>(A.q + row0 * D);
  const char* k = reinterpret_cast<const char*>(A.k + row0 * D);
  r.q0 = *reinterpret_cast<const uint4*>(q + b0);
  r.q1 = *reinterpret_cast<const uint4*>(q + b1);
  r.k0 = *reinterpret_cast<const uint4*>(k + b0);
  r.k1 = *reinterpret_cast<const uint4*>(k + b1);
}
__device__ __forceinline__ void load_raw_gb(Raw& r, const PrefillArgs& A, size_t row0, int nc, int co, int tl) {
  const uint32_t HD2 = (uint32_t)A.n_heads * (D * 2);
  const uint32_t t0 = (uint32_t)min(tl, nc - 1), t1 = (uint32_t)min(16 + tl, nc - 1);
  const uint32_t b0 = t0 * HD2 + 16u * co, b1 = t1 * HD2 + 16u * co;
  const char* gk = reinterpret_cast<const char*>(A.gk + row0 * D);
  const char* beta = reinterpret_cast<const char*>(A.beta + row0);
  const uint32_t H4 = (uint32_t)A.n_heads * 4u;
  r.g0a = *reinterpret_cast<const float4*>(gk + 2u * b0);
  r.g0b = *reinterpret_cast<const float4*>(gk + 2u * b0 + 16u);
  r.g1a = *reinterpret_cast<const float4*>(gk + 2u * b1);
  r.g1b = *reinterpret_cast<const float4*>(gk + 2u * b1 + 16u);
  r.b0 = *reinterpret_cast<const float*>(beta + t0 * H4);
  r.b1 = *reinterpret_cast<const float*>(beta + t1 * H4);
}

// raw v rows of a chunk straight into LDS: 4 rows of 256 bytes per instruction, rows
// 16r + 4w .. 16r + 4w + 3 (r < 2) from wave w of a role; 16-byte chunks land at chunk ^ (2 row & 15)
__device__ __forceinline__ void issue_v(const uint16_t* src, const PrefillArgs& A, uint16_t (&dst)[C][D], size_t row0, int nc, int wu, int lane) {
  const uint16_t* vsrc = src + row0 * D;
  const uint32_t HD = (uint32_t)A.n_heads * D;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int prow = 16 * r + 4 * wu + (lane >> 4);
    const uint32_t e = (uint32_t)min(prow, nc - 1) * HD + 8 * ((lane & 15) ^ ((2 * prow) & 15));
    g2l16(vsrc + e, &dst[16 * r + 4 * wu][0]);
  }
}

// The decay rows of a register set turned, in place, into what stage 1 starts from: gk in log2
// units (0 for tokens past the chunk end, so that G stops advancing there), summed over the tokens
// of each 16-token half up to this lane's. Run in the phase 2 before the set's stage 1, where its
// multiplies and DPP adds fill the time the address unit takes over that phase's loads.
template <int S>
__device__ __forceinline__ void scan_step(float (&x)[8], float (&y)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = x[i] + KDA_ROW_SHR0(x[i], S);
    y[i] = y[i] + KDA_ROW_SHR0(y[i], S);
  }
}
__device__ __forceinline__ void prescan(Raw& r, int nc, int tl) {
  constexpr float kLog2e = 1.4426950408889634f;
  const bool ok0 = tl < nc, ok1 = 16 + tl < nc;
  float gx[8] = {r.g0a.x, r.g0a.y, r.g0a.z, r.g0a.w, r.g0b.x, r.g0b.y, r.g0b.z, r.g0b.w};
  float gy[8] = {r.g1a.x, r.g1a.y, r.g1a.z, r.g1a.w, r.g1b.x, r.g1b.y, r.g1b.z, r.g1b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    gx[i] = ok0 ? gx[i] * kLog2e : 0.f;
    gy[i] = ok1 ? gy[i] * kLog2e : 0.f;
  }
  // the sixteen scans step by step, so that each step's adds are independent of one another
  // (row_scan_add's steps, in its order)
  scan_step<1>(gx, gy);
  scan_step<2>(gx, gy);
  scan_step<4>(gx, gy);
  scan_step<8>(gx, gy);
  r.g0a = make_float4(gx[0], gx[1], gx[2], gx[3]);
  r.g0b = make_float4(gx[4], gx[5], gx[6], gx[7]);
  r.g1a = make_float4(gy[0], gy[1], gy[2], gy[3]);
  r.g1b = make_float4(gy[4], gy[5], gy[6], gy[7]);
}

// What phase 2 of the producer needs from phase 1 to write the chain's operand rows: the
// masked raw q and k (bf16) and the decay factors e^{G_t} and e^{G_31 - G_t} of both tokens.
// eight fp16 products x[i] * y[i], packed
__device__ __forceinline__ uint4 pk8(const float (&x)[8]) {
  return make_uint4(pk_f16(x[0], x[1]), pk_f16(x[2], x[3]), pk_f16(x[4], x[5]), pk_f16(x[6], x[7]));
}
__device__ __forceinline__ uint4 pk8_mul(const float (&x)[8], const float (&y)[8]) {
  return make_uint4(pk_f16(x[0] * y[0], x[1] * y[1]), pk_f16(x[2] * y[2], x[3] * y[3]), pk_f16(x[4] * y[4], x[5] * y[5]),
                    pk_f16(x[6] * y[6], x[7] * y[7]));
}
struct Keep {
  uint4 qt[2], kt[2], kp[2];  // fp16 q e^G, k e^G, k e^{G_31 - G} of tokens lr and 16 + lr
};

// ---------------------------------------------------------------------------
// The factor form below needs every factor in fp32/bf16 range: per key channel, the decay summed
// over the chunk must be at most 60 (log2: 86), so that e^{-G} <= 2^86 and the bf16 low parts of
// q e^G stay normal. It is checked on the chunk's factor e^{G_31} (8 values per lane). Each item
// runs first in the fast form, where a wave with a channel where e^{G_31} < 2^-86, or a decay of
// -inf, only flags the item (its outputs are then overwritten, and its final state is not written);
// a flagged item then runs again in the exact form, where such a wave runs stage1_exact after stage1,
// which rewrites everything stage1 wrote. With the exact path kept out of the fast form's loop, the
// fast form keeps its register allocation and schedule; with it inlined there, a prefill of 1M tokens
// x 96 heads ran 4 % slower although the path was never taken.
constexpr float kMinChunkDecay = 0x1p-86f;  // e^{G_31} below this takes the exact path (e^-59.6)

// producer, phase 1 of the period before chunk c: decay factors and partial A
// and P tiles over this wave's 32 channels. Returns true when the wave's chunk is outside the
// factor form's range (what it wrote is then to be replaced by stage1_exact).
template <class Refill>
__device__ __forceinline__ bool stage1(PrefillLds& L, const Raw& cur, int nc, int b, int pw, int g, int lr, Keep& kp_,
                                       Refill refill) {
  const int co = 4 * pw + g;  // channel octet 8co..8co+7
  const int tl = lr;          // tokens tl (block 0) and 16+tl (block 1)
  const int c8 = 8 * co;
  const bool ok0 = tl < nc, ok1 = 16 + tl < nc;
  // the set's decay rows, already summed within each half by prescan (log2 units)
  const float ps0[8] = {cur.g0a.x, cur.g0a.y, cur.g0a.z, cur.g0a.w, cur.g0b.x, cur.g0b.y, cur.g0b.z, cur.g0b.w};
  const float ps1[8] = {cur.g1a.x, cur.g1a.y, cur.g1a.z, cur.g1a.w, cur.g1b.x, cur.g1b.y, cur.g1b.z, cur.g1b.w};
  if (pw == 0 && g == 0) {
    L.beta[b][tl] = ok0 ? cur.b0 : 0.f;
    L.beta[b][16 + tl] = ok1 ? cur.b1 : 0.f;
  }
  // q and k of tokens past the end are not masked: beta is zero there, so those rows of
  // R and W are exactly zero and the rows drop out of every product (the loads re-read the
  // last token, so the values are finite); gk is masked above so that G stops advancing
  float k0[8], k1[8], q0[8], q1[8];
  unpack_bf16x8(cur.k0, k0); unpack_bf16x8(cur.k1, k1);
  unpack_bf16x8(cur.q0, q0); unpack_bf16x8(cur.q1, q1);
  // q and k are unpacked: their registers take a later chunk's q and k now, so that the address
  // unit works through those loads during this phase's arithmetic (16 rows x 64 bytes per load
  // instruction is slow to address; issued all at once in phase 2 they held the issuing waves for
  // most of it)
  asm volatile("" ::: "memory");
  refill();
  asm volatile("" ::: "memory");
  float e0[8], e1[8], ie0[8], ie1[8], f0[8], f1[8], dl[8];
  // no branch inside this loop: its 32 exponentials are independent across channels and
  // interleave only within one basic block
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // the four exponentials of the prefix sums inside each 16-token half
    const float s0 = ps0[i], s1 = ps1[i];  // log2 of e^{G_t}, e^{G_t - G_15}
    const float p0 = __builtin_amdgcn_exp2f(s0), r0 = __builtin_amdgcn_exp2f(-s0);
    const float p1 = __builtin_amdgcn_exp2f(s1), r1 = __builtin_amdgcn_exp2f(-s1);
    const float T0 = KDA_ROW_BCAST15(p0), T1 = KDA_ROW_BCAST15(p1);   // e^{G_15}, e^{G_31 - G_15}
    e0[i] = p0;                               // e^{G_t}
    e1[i] = T0 * p1;
    ie0[i] = r0;                              // e^{-G_t}
    ie1[i] = KDA_ROW_BCAST15(r0) * r1;        // (lane 15's r0 is e^{-G_15})
    dl[i] = T0 * T1;                          // e^{G_31}
    f0[i] = dl[i] * r0;                       // e^{G_31 - G_t}
    f1[i] = T1 * r1;
  }
  if (tl == 0) {
    *reinterpret_cast<float4*>(&L.dlast[b][c8]) = make_float4(dl[0], dl[1], dl[2], dl[3]);
    *reinterpret_cast<float4*>(&L.dlast[b][c8 + 4]) = make_float4(dl[4], dl[5], dl[6], dl[7]);
  }
  // q e^G and k e^G serve twice: rounded to fp16 they are the chain's operand rows (written to LDS in
  // phase 2), rounded to bf16 they are the row factors of A and P (anchored at the chunk start:
  // A_ij = beta_i sum_c (k_ic e^{G_ic}) (k_jc e^{-G_jc}), P_ti = sum_c (q_tc e^{G_tc}) (k_ic e^{-G_ic}))
  float qe0[8], qe1[8], ke0[8], ke1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { qe0[i] = q0[i] * e0[i]; qe1[i] = q1[i] * e1[i]; ke0[i] = k0[i] * e0[i]; ke1[i] = k1[i] * e1[i]; }
  kp_.qt[0] = pk8(qe0); kp_.qt[1] = pk8(qe1);
  kp_.kt[0] = pk8(ke0); kp_.kt[1] = pk8(ke1);
  kp_.kp[0] = pk8_mul(k0, f0); kp_.kp[1] = pk8_mul(k1, f1);
  // A and P over this wave's 32 channels, straight from registers: lane (g, lr) holds
  // channels 32pw+8g..+7 of tokens lr (block 0) and 16+lr (block 1), which is the
  // A-operand fragment of row lr and the B-operand fragment of column lr
  bf16x8 rk0, rk1, rq0h, rq0l, rq1h, rq1l, ck0h, ck0l, ck1h, ck1l;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    rk0[i] = (__bf16)ke0[i];
    rk1[i] = (__bf16)ke1[i];
    float v = qe0[i];         rq0h[i] = (__bf16)v; rq0l[i] = (__bf16)(v - (float)rq0h[i]);
    v = qe1[i];               rq1h[i] = (__bf16)v; rq1l[i] = (__bf16)(v - (float)rq1h[i]);
    v = k0[i] * ie0[i];       ck0h[i] = (__bf16)v; ck0l[i] = (__bf16)(v - (float)ck0h[i]);
    v = k1[i] * ie1[i];       ck1h[i] = (__bf16)v; ck1l[i] = (__bf16)(v - (float)ck1h[i]);
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
    *reinterpret_cast<f32x4*>(&L.part[pw][tl6][lr][4 * g]) = acc[tl6];
  const float m = __builtin_fminf(__builtin_fminf(__builtin_fminf(dl[0], dl[1]), __builtin_fminf(dl[2], dl[3])),
                                  __builtin_fminf(__builtin_fminf(dl[4], dl[5]), __builtin_fminf(dl[6], dl[7])));
  return __builtin_amdgcn_ballot_w64(m < kMinChunkDecay) != 0;  // (NaN breaks gk <= 0: not caught)
}

// One diagonal 16-block of A and P, summed pairwise in fp32 over this wave's 32 channels: entry
// (i, j), j <= i, is sum_c k_ic k_jc e^{G_ic - G_jc} (q_ic for P), e^{G_i - G_j} = 2^{ps_i - ps_j}
// from the block's inclusive prefix sums ps (log2 units); entries j > i are 0. Lane (g, lr) holds
// channel octet g of token i = lr; row j comes from lane j of the same 16-lane row (a lane shuffle),
// the four octets are added across rows, and one row writes the tile in the partials' [j][i]
// layout. A rolled loop: this path is rare, and its code should not crowd the fast path's.
__device__ __forceinline__ void diag_pairwise(float (&part_a)[16][20], float (&part_p)[16][20], const float (&k)[8],
                                              const float (&q)[8], const float (&ps)[8], int g, int lr) {
  const int lane = threadIdx.x & 63;
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    const int src = (lane & 48) | j;
    float a = 0.f, pp = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float kj = __shfl(k[c], src), pj = __shfl(ps[c], src);
      const float e = (j <= lr) ? __builtin_amdgcn_exp2f(ps[c] - pj) : 0.f;
      const float kje = kj * e;
      a = __builtin_fmaf(k[c], kje, a);
      pp = __builtin_fmaf(q[c], kje, pp);
    }
    a += __shfl_xor(a, 16);
    pp += __shfl_xor(pp, 16);
    a += __shfl_xor(a, 32);
    pp += __shfl_xor(pp, 32);
    if (g == (j & 3)) {
      part_a[j][lr] = a;
      part_p[j][lr] = pp;
    }
  }
}

// producer, phase 1, exact for any decay gk <= 0 (including -inf), for a wave whose chunk is beyond
// the factor form's range; it rewrites everything stage1 wrote (dlast, the operand rows, all six
// partial tiles). The factors at most 1 (e^{G_t}, e^{G_31 - G_t}, e^{G_31}, and the
// off-diagonal tiles' e^{G_t - G_15} of the second half and e^{G_15 - G_t} of the first) are each one
// exponential of a prefix or suffix sum, never a product of a large and a small one; the diagonal
// tiles A00, A11, P00, P11 are summed pairwise; A10 and P10 keep their MFMAs. Decays are clamped at
// 2^-160 per token, which is 0 in fp32, so e^{-inf} = 0 exactly and no sum is infinite.
__device__ __forceinline__ void stage1_exact(PrefillLds& L, const PrefillArgs& A, size_t row0, int nc, int b, int pw,
                                             int g, int lr, Keep& kp_) {
  // the raw registers already hold a later chunk's loads: read this chunk again (this path is rare)
  Raw cur;
  load_raw(cur, A, row0, nc, 4 * pw + g, lr);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  const int co = 4 * pw + g, c8 = 8 * co, tl = lr;
  const bool ok0 = tl < nc, ok1 = 16 + tl < nc;
  constexpr float kLog2e = 1.4426950408889634f;
  float p0[8], p1[8], x0[8], x1[8];  // inclusive prefix and exclusive suffix sums in each half (log2)
  {
    const float gx[8] = {cur.g0a.x, cur.g0a.y, cur.g0a.z, cur.g0a.w, cur.g0b.x, cur.g0b.y, cur.g0b.z, cur.g0b.w};
    const float gy[8] = {cur.g1a.x, cur.g1a.y, cur.g1a.z, cur.g1a.w, cur.g1b.x, cur.g1b.y, cur.g1b.z, cur.g1b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float l0 = ok0 ? __builtin_fmaxf(gx[i] * kLog2e, -160.f) : 0.f;
      const float l1 = ok1 ? __builtin_fmaxf(gy[i] * kLog2e, -160.f) : 0.f;
      p0[i] = row_scan_add(l0);
      p1[i] = row_scan_add(l1);
      x0[i] = row_suffix_excl(l0);
      x1[i] = row_suffix_excl(l1);
    }
  }
  float k0[8], k1[8], q0[8], q1[8];
  unpack_bf16x8(cur.k0, k0); unpack_bf16x8(cur.k1, k1);
  unpack_bf16x8(cur.q0, q0); unpack_bf16x8(cur.q1, q1);
  {
    float e0[8], e1[8], f0[8], f1[8], dl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float B0 = KDA_ROW_BCAST15(p0[i]), B1 = KDA_ROW_BCAST15(p1[i]);  // half totals
      e0[i] = __builtin_amdgcn_exp2f(p0[i]);        // e^{G_t}, first half
      e1[i] = __builtin_amdgcn_exp2f(B0 + p1[i]);   // e^{G_t}, second half
      f0[i] = __builtin_amdgcn_exp2f(x0[i] + B1);   // e^{G_31 - G_t}, first half
      f1[i] = __builtin_amdgcn_exp2f(x1[i]);        // e^{G_31 - G_t}, second half
      dl[i] = __builtin_amdgcn_exp2f(B0 + B1);      // e^{G_31}
    }
    if (tl == 0) {
      *reinterpret_cast<float4*>(&L.dlast[b][c8]) = make_float4(dl[0], dl[1], dl[2], dl[3]);
      *reinterpret_cast<float4*>(&L.dlast[b][c8 + 4]) = make_float4(dl[4], dl[5], dl[6], dl[7]);
    }
    kp_.qt[0] = pk8_mul(q0, e0); kp_.qt[1] = pk8_mul(q1, e1);
    kp_.kt[0] = pk8_mul(k0, e0); kp_.kt[1] = pk8_mul(k1, e1);
    kp_.kp[0] = pk8_mul(k0, f0); kp_.kp[1] = pk8_mul(k1, f1);
  }
  {
    // A10 and P10 on the MFMAs, factored at token 15 into factors at most 1: e^{G_t - G_15} of the
    // second half is 2^{p1}, e^{G_15 - G_t} of the first half is 2^{x0}
    bf16x8 rk1, rq1h, rq1l, ck0h, ck0l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xr1 = __builtin_amdgcn_exp2f(p1[i]), yc0 = __builtin_amdgcn_exp2f(x0[i]);
      rk1[i] = (__bf16)(k1[i] * xr1);
      float v = q1[i] * xr1; rq1h[i] = (__bf16)v; rq1l[i] = (__bf16)(v - (float)rq1h[i]);
      v = k0[i] * yc0;       ck0h[i] = (__bf16)v; ck0l[i] = (__bf16)(v - (float)ck0h[i]);
    }
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const f32x4 a10 = mfma16(rk1, ck0l, mfma16(rk1, ck0h, z4));
    const f32x4 p10 = mfma16(rq1l, ck0h, mfma16(rq1h, ck0l, mfma16(rq1h, ck0h, z4)));
    *reinterpret_cast<f32x4*>(&L.part[pw][2][lr][4 * g]) = a10;
    *reinterpret_cast<f32x4*>(&L.part[pw][5][lr][4 * g]) = p10;
  }
  diag_pairwise(L.part[pw][0], L.part[pw][3], k0, q0, p0, g, lr);  // A00, P00
  diag_pairwise(L.part[pw][1], L.part[pw][4], k1, q1, p1, g, lr);  // A11, P11
}

// producer, phase 2: the fp16 operand rows formed in phase 1 go to LDS (token-major rows lr and 16+lr)
__device__ __forceinline__ void stage1b(PrefillLds& L, const Keep& kp_, int b, int pw, int g, int lr) {
  const int c8 = 8 * (4 * pw + g);
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int t = 16 * blk + lr;
    *reinterpret_cast<uint4*>(&L.qt[b][t][c8]) = kp_.qt[blk];
    *reinterpret_cast<uint4*>(&L.kt[b][t][c8]) = kp_.kt[blk];
    *reinterpret_cast<uint4*>(&L.kp[b][t][c8]) = kp_.kp[blk];
  }
}

// sums of the four channel slices of NTL 16x16 tiles t0..t0+NTL-1: the lane gets rows
// i0..i0+3 of column j of each. All reads are issued before the first sum.
template <int NTL>
__device__ __forceinline__ void reduce_tiles(const PrefillLds& L, int t0, int j, int i0, f32x4 (&s4)[NTL]) {
  f32x4 pv[NTL][4];
#pragma unroll
  for (int tile = 0; tile < NTL; ++tile)
#pragma unroll
    for (int w = 0; w < 4; ++w) pv[tile][w] = *reinterpret_cast<const f32x4*>(&L.part[w][t0 + tile][j][i0]);
#pragma unroll
  for (int tile = 0; tile < NTL; ++tile) {
    s4[tile] = pv[tile][0];
#pragma unroll
    for (int w = 1; w < 4; ++w)
#pragma unroll
      for (int r = 0; r < 4; ++r) s4[tile][r] += pv[tile][w][r];
  }
}

// phase 2, on one chain wave per block: diagonal 16-block blk of A (the beta-scaled strict lower part
// of the summed tile) and of X = (I + A)^-1. The off-diagonal block of X is never formed: the chain
// applies it as W1 = X11 (R1 - A10 W0). The two blocks are independent and go to two waves.
__device__ __forceinline__ void stage2_solve(PrefillLds& L, int b, int lane, int blk) {
  const int g = lane >> 4, lr = lane & 15;
  {
    const int j = lane >> 2, i0 = 4 * (lane & 3);
    f32x4 sums[1];
    reduce_tiles<1>(L, blk, j, i0, sums);  // tile 0: A00, tile 1: A11
    const f32x4 s4 = sums[0];
    const float4 b4 = *reinterpret_cast<const float4*>(&L.beta[b][16 * blk + i0]);
    const int jg = 16 * blk + j, ig = 16 * blk + i0;
    L.ar[ig][jg] = (jg < ig) ? s4[0] * b4.x : 0.f;
    L.ar[ig + 1][jg] = (jg < ig + 1) ? s4[1] * b4.y : 0.f;
    L.ar[ig + 2][jg] = (jg < ig + 2) ? s4[2] * b4.z : 0.f;
    L.ar[ig + 3][jg] = (jg < ig + 3) ? s4[3] * b4.w : 0.f;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  // Forward substitution on rows. DPP row g of the wave (16 lanes) holds the columns q with
  // q % 4 == g of the block, lane lr = row i: x[m] = X[i][4m + g]. Step kk subtracts A[i][kk]
  // times row kk, which row_newbcast:kk reads from lane kk of the same DPP row; row kk has no
  // entries right of column kk, so columns beyond kk are skipped. Every X[i][q] takes the same
  // sequence of fused multiply-adds whichever lane holds it.
  const int par = g, i = lr;
  float arow[16];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const float4 t4 = *reinterpret_cast<const float4*>(&L.ar[16 * blk + i][16 * blk + 4 * q4]);
    arow[4 * q4] = -t4.x; arow[4 * q4 + 1] = -t4.y; arow[4 * q4 + 2] = -t4.z; arow[4 * q4 + 3] = -t4.w;
  }
  float x[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) x[m] = (4 * m + par == i) ? 1.f : 0.f;
#define KDA_SOLVE_STEP(kk)                                                                                  \
  _Pragma("unroll") for (int m = 0; 4 * m <= (kk); ++m) {                                                   \
    const float xk_ = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[m]), 0x150 + (kk), 0xf, 0xf, true)); \
    x[m] = __builtin_fmaf(arow[kk], xk_, x[m]);                                                             \
  }
  KDA_SOLVE_STEP(0) KDA_SOLVE_STEP(1) KDA_SOLVE_STEP(2) KDA_SOLVE_STEP(3) KDA_SOLVE_STEP(4)
  KDA_SOLVE_STEP(5) KDA_SOLVE_STEP(6) KDA_SOLVE_STEP(7) KDA_SOLVE_STEP(8) KDA_SOLVE_STEP(9)
  KDA_SOLVE_STEP(10) KDA_SOLVE_STEP(11) KDA_SOLVE_STEP(12) KDA_SOLVE_STEP(13) KDA_SOLVE_STEP(14)
#undef KDA_SOLVE_STEP
#pragma unroll
  for (int m = 0; m < 4; ++m)
    L.xb[b][16 * blk + i][16 * blk + 4 * m + par] = __builtin_bit_cast(uint16_t, (_Float16)x[m]);
}

// producer wave 2, phase 2: -A10 = -(beta-scaled summed tile), fp16, for the chain's W1
__device__ __forceinline__ void stage2_a10(PrefillLds& L, int b, int lane) {
  const int j = lane >> 2, i0 = 4 * (lane & 3);
  f32x4 sums[1];
  reduce_tiles<1>(L, 2, j, i0, sums);
  const float4 b4 = *reinterpret_cast<const float4*>(&L.beta[b][16 + i0]);
  const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) L.an[b][i0 + r][j] = __builtin_bit_cast(uint16_t, (_Float16)(-sums[0][r] * bv[r]));
}

// producer wave 1, phase 2: P = lower part (diagonal included) of the summed tiles, fp16
__device__ __forceinline__ void stage2_p(PrefillLds& L, int b, int lane) {
  const int j = lane >> 2, i0 = 4 * (lane & 3);
  f32x4 sums[3];
  reduce_tiles<3>(L, 3, j, i0, sums);
#pragma unroll
  for (int tile = 3; tile < 6; ++tile) {  // P00, P11, P10
    const int I = tile == 3 ? 0 : 1, J = tile == 4 ? 1 : 0;
    const f32x4 s4 = sums[tile - 3];
    const int jg = 16 * J + j;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ig = 16 * I + i0 + r;
      L.pm[b][ig][jg] = (jg <= ig) ? __builtin_bit_cast(uint16_t, (_Float16)s4[r]) : (uint16_t)0;
    }
  }
}

// GATED: the output gated RMSNorm replaces the store of o (whole-chain items only): phase 1 keeps o in
// registers and writes each token's slice sums of squares; the next period's phase 1 (or the item's
// end, for its last chunk) adds them in slice order and writes y in bf16.
template <bool GATED>
__global__ void __launch_bounds__(NT) prefill_kernel(PrefillArgs A) {
  __shared__ PrefillLds L;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, lr = lane & 15;  // MFMA lane group and lane row/column
  const bool producer = wave >= 4;          // wave-uniform role
  const int rw = wave & 3;                  // wave index within the role
  const int rwu = __builtin_amdgcn_readfirstlane(rw);
  const int H = A.n_heads;

  // constant zero blocks: P is lower triangular in 16-blocks
  for (int e = tid; e < 2 * 16 * 16; e += NT) {
    const int b = e >> 8, i = (e >> 4) & 15, j = 16 + (e & 15);
    L.pm[b][i][j] = 0;
  }
  if constexpr (GATED) {
    for (int i = tid; i < D; i += NT) L.nw[i] = A.norm_w[i];
  }

  // A workgroup's first item is fixed: within each 16 workgroups, b and b + 8 (the same XCD under
  // the dispatcher's round-robin placement) take work-list positions 2j and 2j + 1, which a plan
  // with two value blocks fills with the two halves of one chain, so that the second half's reads
  // of q, k, gk and beta find the first half's in that XCD's L2. Later items come from the counter.
  const int G = (int)gridDim.x, b0 = (int)blockIdx.x;
  int first = b0;
  if (b0 < G - G % 16) first = 2 * (8 * (b0 >> 4) + (b0 & 7)) + ((b0 >> 3) & 1);
  for (int round = 0;; ++round) {
    __syncthreads();
    if (tid == 0) {
      L.item = round == 0 ? first : atomicAdd(&A.ws->counter, 1) + G;
      L.redo = 0;
    }
    __syncthreads();
    const int it = L.item;
    if (it < 0 || it >= A.n_items) break;  // also ends a launch on a stale counter
    const int4 wi = A.items[it];
    const int n = wi.x, h = wi.y & 0xffff, vb = wi.y >> 16;  // head, value block
    const int64_t tok0 = wi.z;
    const int len = wi.w;
    if (n < 0 || n >= A.n_seq || h >= H || vb < 0 || vb >= A.n_vblk || tok0 < 0 || len < 0 || tok0 + len > A.total_tokens)
      continue;
    const size_t unit = (size_t)n * H + h;
    const int nch = (len + C - 1) / C;

    // pass 0 runs the item in the fast form; pass 1, only for an item that pass 0 flagged, runs it
    // again in the exact form. The flag is set before some barrier of pass 0 and read by every wave
    // after its last one, so all waves take the same decision.
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == 1 && !L.redo) break;

      // Both roles run nch + 1 periods of two barriers each. Period p runs the
      // chain of chunk p (p >= 0) beside the preparation of chunk p + 1.
      // Inside each role the lane index is made opaque once per item, so that the compiler
      // cannot hoist one role's lane-dependent addresses out of the item loop, where they would
      // stay live (and spill) while the other role runs.
      int lane_o = lane;
      asm volatile("" : "+v"(lane_o));
      const int g_o = lane_o >> 4, lr_o = lane_o & 15;
      if (producer) {
        const int pw = rw;
        const int lane = lane_o, g = g_o, lr = lr_o;
        auto produce = [&](auto exact_form) {
          constexpr bool EXACT = decltype(exact_form)::value;
          // Raw inputs are prefetched two periods ahead: q, k, gk, beta into registers, alternating
          // between two sets (chunk c lives in set c & 1 from the period that issues it, c - 3,
          // until its stage 1 in period c - 1: its q and k in that period's phase 1, as soon as stage 1
          // has unpacked the set's previous q and k, its gk and beta in phase 2; in phase 2 of period
          // c - 2 prescan turns its gk into the prefix sums stage 1 starts from), and v straight into
          // vr[c & 1] (issued in period c - 2, read by the chain in period c; with GATED the gate rows
          // go into gr[c & 1] the same way). Every period issues the same 12 loads (14 with GATED; past
          // the last chunk they re-read it), so the compiler's waits before each register use count
          // exactly, and the wait that closes a period can leave just that period's loads in flight.
          if (nch == 0) {
            __syncthreads();
            __syncthreads();
          } else {
            Raw ra, rb;
            auto issue = [&](Raw& r, int c) {
              c = min(c, nch - 1);
              load_raw(r, A, (size_t)(tok0 + C * c) * H + h, min(C, len - C * c), 4 * pw + g, lr);
            };
            auto issue_early = [&](Raw& r, int c) {
              c = min(c, nch - 1);
              load_raw_qk(r, A, (size_t)(tok0 + C * c) * H + h, min(C, len - C * c), 4 * pw + g, lr);
            };
            auto issue_late = [&](Raw& r, int c) {
              c = min(c, nch - 1);
              load_raw_gb(r, A, (size_t)(tok0 + C * c) * H + h, min(C, len - C * c), 4 * pw + g, lr);
            };
            auto issue_vc = [&](int c) {
              c = min(c, nch - 1);
              issue_v(A.v, A, L.vr[c & 1], (size_t)(tok0 + C * c) * H + h, min(C, len - C * c), pw, lane);
              if constexpr (GATED) issue_v(A.gate, A, L.gr[c & 1], (size_t)(tok0 + C * c) * H + h, min(C, len - C * c), pw, lane);
            };
            issue(ra, 0);
            asm volatile("" ::: "memory");  // keep the issue order: set a, v of chunk 0, set b
            issue_vc(0);
            asm volatile("" ::: "memory");
            issue(rb, 1);
            asm volatile("" ::: "memory");
            auto nc_of = [&](int c) { c = min(c, nch - 1); return min(C, len - C * c); };
            prescan(ra, nc_of(0), lr);
            auto period = [&](int p, Raw& use, Raw& other) {
              const int c1 = p + 1, b1 = c1 & 1;
              Keep keep;
              if (c1 < nch) {
                const int ncc = min(C, len - C * c1);
                if (stage1(L, use, ncc, b1, pw, g, lr, keep, [&] { issue_early(use, c1 + 2); })) {
                  if constexpr (EXACT) stage1_exact(L, A, (size_t)(tok0 + C * c1) * H + h, ncc, b1, pw, g, lr, keep);
                  else L.redo = 1;
                }
              } else {
                issue_early(use, c1 + 2);
              }
              __syncthreads();
              issue_late(use, c1 + 2);
              __builtin_amdgcn_sched_barrier(0);
              prescan(other, nc_of(c1 + 1), lr);  // the next period's set, while the loads above go out
              __builtin_amdgcn_sched_barrier(0);
              issue_vc(c1 + 1);  // into the buffer the chain read in this period's phase 1
              if (c1 < nch) stage1b(L, keep, b1, pw, g, lr);
              // everything older than this period's 12 (14) loads has landed: the next chunk's
              // register set and the v (and gate) rows the chain reads in the next period
              if constexpr (GATED) __builtin_amdgcn_s_waitcnt(0x0f7e);  // vmcnt(14): the gate rows are 2 more loads
              else __builtin_amdgcn_s_waitcnt(0x0f7c);                  // vmcnt(12)
              __syncthreads();
            };
            // periods -1 .. nch-1 in pairs, so that both sets' loads are issued on every path
            // around the loop
            int p = -1;
            for (; p + 1 < nch; p += 2) {
              period(p, ra, rb);
              period(p + 1, rb, ra);
            }
            if (p < nch) period(p, ra, rb);
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no LDS write may outlive the item
          }
        };
        if (pass == 0) produce(std::false_type{});
        else produce(std::true_type{});
      } else {
        const int lane = lane_o, g = g_o, lr = lr_o;
        // The chain on the item's value columns: all 128 (four waves of 32, NV = 2 tiles of 16), or
        // one of two halves of 64 (four waves of 16, NV = 1). Each 16-column tile runs the same
        // instructions either way, so a split item gives the same bits as the whole one.
        auto chain = [&](auto nv_tiles) {
          constexpr int NV = decltype(nv_tiles)::value;
          const int cw = rw;
          const int cb = vb * (D / 2) * (2 - NV) + 16 * NV * cw;  // first value column of this wave
          // This lane's element of a row-major [128][128] state tile is (16mc+4g+r, cb+16nv+lr), at
          // tile + soff + (16mc+r)*D + 16nv. soff is made opaque here so that the compiler keeps one
          // offset per lane instead of hoisting all the element offsets out of the item loop.
          int soff = 4 * g * D + cb + lr;
          asm volatile("" : "+v"(soff));
          // state slice of this wave in accumulator layout: S[mc][nv] holds rows 16mc+4g+r, column cb+16nv+lr
          f32x4 S[8][NV];
          if (A.state_in) {
            const float* src = A.state_in + unit * D * D + soff;
    #pragma unroll
            for (int mc = 0; mc < 8; ++mc)
    #pragma unroll
              for (int nv = 0; nv < NV; ++nv)
    #pragma unroll
                for (int r = 0; r < 4; ++r) S[mc][nv][r] = src[(16 * mc + r) * D + 16 * nv];
          } else {
    #pragma unroll
            for (int mc = 0; mc < 8; ++mc)
    #pragma unroll
              for (int nv = 0; nv < NV; ++nv) S[mc][nv] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          f16x8 Wh[NV], Wl[NV];

          // GATED: o of tokens lr and 16 + lr of the last chunk and their gate bits (columns c0 .. c0 + 3),
          // kept in registers from the phase 1 that forms them to the next period's phase 1, where the
          // output gated RMSNorm of that chunk runs just before the new o replaces them. Its stores then
          // go out late in phase 1, as the plain path's stores of o do: in phase 2, or early in phase 1,
          // they would wait behind the producers' burst of loads in a full memory queue
          f32x4 Og[2][NV];
          uint2 Gq[2][NV];
          auto norm_epilogue = [&](int pc) {
            if constexpr (GATED && NV == 2) {
              // rows past the chunk end fall outside the buffer range and are dropped by the hardware
              const int ncc = min(C, len - C * pc);
              const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
                  A.y + ((size_t)(tok0 + C * pc) * H + h) * D, 0, (int)((((uint32_t)ncc - 1) * H * D + D) * 2), 0x00020000);
    #pragma unroll
              for (int mt = 0; mt < 2; ++mt) {
                const uint32_t t = 16 * mt + lr;
                const float rstd = L.rs[t];
    #pragma unroll
                for (int nv = 0; nv < 2; ++nv) {
                  const float4 w4 = *reinterpret_cast<const float4*>(&L.nw[cb + 16 * nv + 4 * g]);
                  const uint2 yv = norm_apply4(Og[mt][nv], Gq[mt][nv], w4, rstd);
                  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2v, yv), yrs,
                                                        (int)((t * H * D + cb + 16 * nv + 4 * g) * 2), 0, 0);
                }
              }
            }
          };

          for (int p = -1; p < nch; ++p) {
            const int b = p & 1;
            const int nc = min(C, len - C * p);
            if (p >= 0) {
              // ---------------- Kt S0 and Qt S0 ----------------
              // S enters as fp16 B operands: step s reduces over rows {16(2s)+4g+r} then {16(2s+1)+4g+r},
              // and the A operands read the same permutation of their columns
              // The same fragments serve as the A operand of S^T, so (Qt S0)^T = S0^T Qt^T comes out
              // transposed: QT[nv][mt] holds rows = value columns, columns = tokens.
              f32x4 KS[2][NV], QT[NV][2];
    #pragma unroll
              for (int mt = 0; mt < 2; ++mt)
    #pragma unroll
                for (int nv = 0; nv < NV; ++nv) { KS[mt][nv] = f32x4{0.f, 0.f, 0.f, 0.f}; QT[nv][mt] = f32x4{0.f, 0.f, 0.f, 0.f}; }
    #pragma unroll
              for (int s = 0; s < 4; ++s) {
                f16x8 sh[NV];
    #pragma unroll
                for (int nv = 0; nv < NV; ++nv) sh[nv] = to_h8(S[2 * s][nv], S[2 * s + 1][nv]);
    #pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                  const int m = 16 * mt + lr;
                  const f16x8 kr = perm_h(&L.kt[b][m][32 * s], g);
                  const f16x8 qr = perm_h(&L.qt[b][m][32 * s], g);
    #pragma unroll
                  for (int nv = 0; nv < NV; ++nv) {
                    KS[mt][nv] = mfma_h(kr, sh[nv], KS[mt][nv]);
                    QT[nv][mt] = mfma_h(sh[nv], qr, QT[nv][mt]);
                  }
                }
              }
              // ---------------- R = diag(beta)(V - Kt S0), W = X R ----------------
              // by blocks: W0 = X00 R0, W1 = X11 (R1 - A10 W0), 16x16x16 MFMAs with fp16 hi + lo operands
              f32x4 W[2][NV];
              const float mone = minus_one();
              {
                const f16x4 x00 = __builtin_bit_cast(f16x4, lds8(&L.xb[b][lr][4 * g]));
                const f16x4 x11 = __builtin_bit_cast(f16x4, lds8(&L.xb[b][16 + lr][16 + 4 * g]));
                const f16x4 a10 = __builtin_bit_cast(f16x4, lds8(&L.an[b][lr][4 * g]));
    #pragma unroll
                for (int nv = 0; nv < NV; ++nv) {
                  f32x4 R[2];
                  const int c0 = cb + 16 * nv + 4 * (lr & 3);
    #pragma unroll
                  for (int mt = 0; mt < 2; ++mt) {
                    // V[16mt+4g+r][32cw+16nv+lr] through the transposing read of the swizzled raw rows;
                    // the four rows of one read land in four different 8-bank groups
                    const int row = 16 * mt + 4 * g + (lr >> 2);
                    const uint2 vv = lds_tr(&L.vr[b][row][8 * ((c0 >> 3) ^ ((2 * row) & 15)) + (c0 & 7)]);
                    const float4 b4 = *reinterpret_cast<const float4*>(&L.beta[b][16 * mt + 4 * g]);
                    R[mt][0] = b4.x * (bf2f(vv.x & 0xffffu) - KS[mt][nv][0]);
                    R[mt][1] = b4.y * (bf2f(vv.x >> 16) - KS[mt][nv][1]);
                    R[mt][2] = b4.z * (bf2f(vv.y & 0xffffu) - KS[mt][nv][2]);
                    R[mt][3] = b4.w * (bf2f(vv.y >> 16) - KS[mt][nv][3]);
                  }
                  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
                  f16x4 hi, lo;
                  split_h4(R[0], hi, lo, mone);
                  f32x4 w0 = mfma_h16(x00, lo, mfma_h16(x00, hi, z4));
                  split_h4(w0, hi, lo, mone);
                  f32x4 r1 = mfma_h16(a10, lo, mfma_h16(a10, hi, R[1]));
                  split_h4(r1, hi, lo, mone);
                  W[0][nv] = w0;
                  W[1][nv] = mfma_h16(x11, lo, mfma_h16(x11, hi, z4));
                }
              }
    #pragma unroll
              for (int nv = 0; nv < NV; ++nv) split_h8(W[0][nv], W[1][nv], Wh[nv], Wl[nv], mone);
              if (p >= 1) norm_epilogue(p - 1);  // (GATED only) the previous chunk's output, before its o is replaced

              // ---------------- O^T = scale (S0^T Qt^T + W^T P^T), stored from the accumulators ----------------
              // lane (g, lr) holds O[16mt + lr][cb + 16nv + 4g + r], r < 4: one 16-byte store per tile
    #pragma unroll
              for (int mt = 0; mt < 2; ++mt) {
                const f16x8 pa = perm_h(&L.pm[b][16 * mt + lr][0], g);
                const int t = 16 * mt + lr;
                float* orow = A.o + ((size_t)(tok0 + C * p) * H + h) * D + ((uint32_t)t * H * D + cb + 4 * g);
    #pragma unroll
                for (int nv = 0; nv < NV; ++nv) {
                  f32x4 acc = QT[nv][mt];
                  acc = mfma_h(Wh[nv], pa, acc);
                  acc = mfma_h(Wl[nv], pa, acc);
                  if constexpr (GATED) {
                    Og[mt][nv] = f32x4{A.scale * acc[0], A.scale * acc[1], A.scale * acc[2], A.scale * acc[3]};
                    const int c0 = cb + 16 * nv + 4 * g;
                    Gq[mt][nv] = *reinterpret_cast<const uint2*>(&L.gr[b][t][8 * ((c0 >> 3) ^ ((2 * t) & 15)) + (c0 & 7)]);
                  } else if (t < nc) {
                    *reinterpret_cast<float4*>(orow + 16 * nv) = make_float4(A.scale * acc[0], A.scale * acc[1], A.scale * acc[2], A.scale * acc[3]);
                  }
                }
                // this lane's slice (4 cw + g) of token t: columns 32 cw + 4 g + {0..3}, then + 16
                if constexpr (GATED && NV == 2) L.ssq[t][4 * cw + g] = norm_slice_ssq(Og[mt][0], Og[mt][1]);
              }
            }
            // The state update reads only this chunk's K' rows and e^{G_31} (written by the preparation
            // waves in the previous period) and this wave's own W, so it runs before the barrier, in the
            // time the chain would otherwise wait there for the preparation of the next chunk.
            if (p >= 0) {
              // ---------------- S = e^{G_31} S0 + K'^T W ----------------
    #pragma unroll
              for (int mc = 0; mc < 8; ++mc) {
                const float4 d4 = *reinterpret_cast<const float4*>(&L.dlast[b][16 * mc + 4 * g]);
                // K'^T rows 16mc+lr, reduction positions t = 4g+r and 16+4g+r, via the transposing read
                const uint16_t* base = &L.kp[b][4 * g + (lr >> 2)][16 * mc + 4 * (lr & 3)];
                const f16x8 ka = as_f16x8(lds_tr(base), lds_tr(base + 16 * TM));
    #pragma unroll
                for (int nv = 0; nv < NV; ++nv) {
                  f32x4 acc = S[mc][nv];
                  acc[0] *= d4.x; acc[1] *= d4.y; acc[2] *= d4.z; acc[3] *= d4.w;
                  acc = mfma_h(ka, Wh[nv], acc);
                  acc = mfma_h(ka, Wl[nv], acc);
                  S[mc][nv] = acc;
                }
              }

              // ---------------- snapshot at chunk ends q with q % interval == 0 ----------------
              const int q = C * p + nc;
              if (A.snap_interval > 0 && q % A.snap_interval == 0) {
                const int m = q / A.snap_interval;
                float* dst = A.snap + (((size_t)n * A.snap_slots + (m - 1) % A.snap_slots) * H + h) * D * D + soff;
    #pragma unroll
                for (int mc = 0; mc < 8; ++mc)
    #pragma unroll
                  for (int nv = 0; nv < NV; ++nv)
    #pragma unroll
                    for (int r = 0; r < 4; ++r) dst[(16 * mc + r) * D + 16 * nv] = S[mc][nv][r];
              }
            }
            __syncthreads();
            // (GATED) 1 / rms of each of this chunk's token rows from the slice sums of phase 1, on the
            // chain wave with the most slack in phase 2; the next period's phase 1 uses them
            if constexpr (GATED && NV == 2) {
              if (cw == 3 && p >= 0 && lane < C) {
                float ss = 0.f;  // the 16 slice sums, in slice order
    #pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                  const float4 s4 = *reinterpret_cast<const float4*>(&L.ssq[lane][4 * k4]);
                  ss = ss + s4.x;
                  ss = ss + s4.y;
                  ss = ss + s4.z;
                  ss = ss + s4.w;
                }
                L.rs[lane] = norm_rstd(ss, A.eps);
              }
            }
            // the next chunk's X, P and -A10 from the partials the producers wrote in phase 1, on the
            // chain waves (the producers' phase 2 is taken up by issuing the next loads)
            if (cw == 0 && p + 1 < nch) stage2_solve(L, (p + 1) & 1, lane, 0);
            else if (cw == 1 && p + 1 < nch) stage2_p(L, (p + 1) & 1, lane);
            else if (cw == 2 && p + 1 < nch) stage2_a10(L, (p + 1) & 1, lane);
            else if (cw == 3 && p + 1 < nch) stage2_solve(L, (p + 1) & 1, lane, 1);
            __syncthreads();
          }

          if (nch >= 1) norm_epilogue(nch - 1);  // (GATED only) the last chunk's output

          // a flagged fast pass leaves the final state unwritten, so that pass 1 still finds the
          // initial state where the caller passed the same buffer for both
          if (pass == 1 || !L.redo) {
            float* dst = A.state_out + unit * D * D + soff;
    #pragma unroll
            for (int mc = 0; mc < 8; ++mc)
    #pragma unroll
              for (int nv = 0; nv < NV; ++nv)
    #pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * mc + r) * D + 16 * nv] = S[mc][nv][r];
          }

        };
        if (GATED || A.n_vblk == 1) chain(std::integral_constant<int, 2>{});
        else chain(std::integral_constant<int, 1>{});
        if (A.snap_count && h == 0 && vb == 0 && tid == 0) A.snap_count[n] = A.snap_interval > 0 ? len / A.snap_interval : 0;
      }
    }
  }

  // the last workgroup out resets the counters, so a later launch with the
  // same resident work list starts from zero. No fence is needed: every
  // workgroup's last draw from the counter has returned its value (the loop
  // above ended on it) before its increment of `done` is issued, so when the
  // last increment returns, no draw of this launch is still to be performed.
  // (A release fence here would also write back this XCD's L2 once per
  // workgroup, a few microseconds at the end of the launch.)
  if (tid == 0) {
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
  return cus[device];  // one workgroup per CU (LDS-bound)
}

hipError_t launch_prefill(const PrefillArgs& a, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (a.y) hipLaunchKernelGGL(prefill_kernel<true>, dim3(grid), dim3(NT), 0, stream, a);
  else hipLaunchKernelGGL(prefill_kernel<false>, dim3(grid), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
