// kda_internal.h -- argument blocks and launchers shared by the libkda translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// sets the thread-local text behind kda_last_error and returns s (defined in kda_api.cpp)
kda_status fail(kda_status s, const char* msg);
inline kda_status ok() { return KDA_OK; }

struct VerifyArgs {
  int batch, n_tok, n_heads, n_layers, layer, n_slots;
  const void* q;
  const void* k;
  const void* v;
  const float* gk;
  const float* beta;
  const float* state_pool;
  const int32_t* slot_idx;
  float* o;
  void* ring_k;  // nullptr: nothing recorded
  void* ring_v;
  float* ring_gk;
  float* ring_beta;
  int ring_len;
  const int32_t* ring_start;  // nullptr: 0
  const int32_t* commit_len;  // nullptr: no commit
  float* commit_pool;
  float scale;
  // fused fold-then-verify (nullptr fold_len: plain verify): fold fold_len[b] entries of the
  // previous window, at ring positions fold_start[b] + i, into fold_pool (== state_pool) first
  const int32_t* fold_len;
  const int32_t* fold_start;  // nullptr: 0
  float* fold_pool;
  // ragged windows (nullptr cu_tok: every request has n_tok tokens at rows b * n_tok + t): request
  // b's window is rows [cu_tok[b], cu_tok[b + 1]) of total_tok, clamped, at most n_tok long
  const int32_t* cu_tok;
  int total_tok;
};

struct FoldArgs {
  int batch, n_heads, n_layers, n_slots;
  float* state_pool;
  const int32_t* slot_idx;
  const void* ring_k;
  const void* ring_v;
  const float* ring_gk;
  const float* ring_beta;
  int ring_len;
  const int32_t* ring_start;
  const int32_t* accepted_len;
};

// Work list header at the start of the prefill workspace.
struct PrefillWsHeader {
  int32_t counter;  // next item to take
  int32_t done;     // workgroups finished
  int32_t pad[62];  // items start at byte 256
};

struct PrefillArgs {
  int n_seq, n_heads, n_items;
  int64_t total_tokens;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* gk;
  const float* beta;
  const float* state_in;  // nullptr: zeros
  float* state_out;
  float* o;
  float* snap;  // nullptr: none
  int snap_slots;
  int snap_interval;  // 0: none
  int32_t* snap_count;
  PrefillWsHeader* ws;
  const int4* items;  // (sequence, head | value block << 16, first token, length)
  int n_vblk;         // value blocks per (sequence, head): 1 (all 128 columns) or 2 (halves)
  float scale;
  // the fused output gated RMSNorm (y != nullptr, whole-chain items only): y replaces o
  const uint16_t* gate;  // bf16 [T, H, 128]
  const float* norm_w;   // fp32 [128]
  float eps;
  uint16_t* y;           // bf16 [T, H, 128]
};

// the KDA prologue: short conv + SiLU (+ L2 norm for q, k), beta sigmoid, gk = -softplus
struct PrologueArgs {
  int n_seq, n_heads, conv_width;
  int64_t total_tokens;
  const int32_t* cu_seqlens;  // [n_seq + 1], read clamped
  const uint16_t* xq;         // bf16 [T, H, 128] projections
  const uint16_t* xk;
  const uint16_t* xv;
  const float* conv_w;        // fp32 [3, H * 128, W]
  const uint16_t* state_in;   // bf16 [n_seq, 3, W - 1, H * 128] or nullptr (zeros)
  uint16_t* state_out;        // same layout or nullptr (not written)
  const float* b_raw;         // fp32 [T, H]
  const float* g_raw;         // fp32 [T, H, 128]
  float eps;
  uint16_t* q;                // bf16 [T, H, 128]
  uint16_t* k;
  uint16_t* v;
  float* beta;                // fp32 [T, H]
  float* gk;                  // fp32 [T, H, 128]
};
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream);

// one fused decode step (prologue + recurrent step with in-place commit + output gated RMSNorm)
struct DecodeArgs {
  int batch, n_heads, n_layers, layer, n_slots, conv_width;
  const uint16_t* xq;  // bf16 [B, H, 128] each
  const uint16_t* xk;
  const uint16_t* xv;
  const float* conv_w;   // fp32 [3, H * 128, W]
  uint16_t* conv_state;  // bf16 [B, 3, W - 1, H * 128], in place
  const float* b_raw;    // fp32 [B, H]
  const float* g_raw;    // fp32 [B, H, 128]
  float* state_pool;     // fp32 [n_slots, L, H, 128, 128], the commit in place
  const int32_t* slot_idx;
  const uint16_t* gate;  // bf16 [B, H, 128]
  const float* norm_w;   // fp32 [128]
  float qk_eps, norm_eps, scale;
  uint16_t* y;  // bf16 [B, H, 128]
  float* o;     // fp32 [B, H, 128] or nullptr
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_state_move(int n_moves, const kda_move* moves, int n_slots, int64_t slot_floats, float* pool,
                             hipStream_t stream);

hipError_t launch_verify(const VerifyArgs& a, bool f32_inputs, hipStream_t stream);
// the output gated RMSNorm on its own: rows of 128 fp32 values -> bf16
hipError_t launch_gated_rmsnorm(int64_t rows, const float* o, const uint16_t* gate, const float* w, float eps,
                                uint16_t* y, hipStream_t stream);
// chunked-form verify on the matrix cores: bf16 inputs, n_tok <= 16, no recurrent commit
bool verify_chunk_eligible(const VerifyArgs& a, bool f32_inputs);
hipError_t launch_verify_chunk(const VerifyArgs& a, hipStream_t stream);
// fused fold-then-verify: bf16 inputs, n_tok <= 8, ring of at most 16 entries
hipError_t launch_fold_verify(const VerifyArgs& a, hipStream_t stream);
hipError_t launch_fold(const FoldArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int grid, hipStream_t stream);
int prefill_max_grid(int device);
// measurement probes (kda_probe.hip): streaming copy and read of n_f4 float4s, a loop of bf16 MFMAs
hipError_t launch_probe_copy(const void* src, void* dst, int64_t n_f4, int grid, hipStream_t stream);
hipError_t launch_probe_read(const void* src, int64_t n_f4, float* sink, int grid, hipStream_t stream);
hipError_t launch_probe_mfma(int iters, int grid, float seed, float* sink, hipStream_t stream);

}  // namespace kda
