/*
 * kda.h -- C ABI of libkda, the MI355X (gfx950) library for the KDA (Kimi
 * Delta Attention) gated delta-rule recurrence.
 *
 * The recurrence, per (sequence or request slot, layer, head), with key and
 * value head dimension K = V = 128 and an fp32 state S[K][V] (key channel =
 * row index):
 *
 *   a[c]    = exp(gk[t][c])                        per-key-channel decay, gk <= 0
 *   u[j]    = sum_c a[c] k[t][c] S[c][j]           prediction of the decayed state
 *   w[j]    = beta[t] (v[t][j] - u[j])             delta-rule error
 *   S[c][j] = a[c] S[c][j] + k[t][c] w[j]          decay, then rank-1 update, in place
 *   o[t][j] = scale * sum_c q[t][c] S[c][j]        readout from the updated state
 *
 * Sources (page title, section):
 *  [LMSYS-MEM] "SGLang and Miles Add Day-0 Support for Kimi K3" (LMSYS
 *      blog), section "Hybrid KDA Memory Management": one fixed-size
 *      recurrent state per request, overwritten in place every token;
 *      subsection "Three state moves on the forward stream": snapshots at
 *      chunk boundaries into a ping-pong "extra buffer", every state copy
 *      ordered on the one forward stream.
 *  [LMSYS-RSSM] same post, section "ReplaySSM: raw-input replay for the KDA
 *      state": a K x V state (64 KB at K = V = 128); verify reads the
 *      committed checkpoint and never writes it, and stores each step's raw
 *      inputs (v, k, gk, beta), about 1 KB; one fold launch over every layer
 *      and head replays only the accepted prefix in place, using the stored
 *      gate values, bit-identical to the recurrent commit.
 *  [B200-FKDA] Kimi K3 B200 deployment notes (zdszero.github.io), FlashKDA
 *      items of the optimisation timeline: one fused kernel per chunk with
 *      intermediates on chip; an fp32 [128,128] state per (sequence, head);
 *      persistent launch and longest-first (LPT) order of sequences; a CPU
 *      split plan built once per batch from host data and reused by every
 *      layer, with no device read-back.
 *  [B200-RING] same notes, section "DSPARK and KDA state" (decode-side
 *      choices): a small ring per slot holding (v, k, gate, beta); its length
 *      is a power of two and at least 2 * (gamma + 1). The same list names
 *      the two verify layouts: static (every request verifies all gamma + 1
 *      tokens) and ragged (windows trimmed per request by confidence).
 *  [B200-NORM] same notes, prefill / decode kernel-fusion items: the KDA
 *      output passes through a gated RMSNorm that reads the attention output
 *      at its native stride; that norm is the one fusion allowed fast math
 *      (tolerance 8e-3). The formula is not printed; the reading used here is
 *      RMSNorm over the head's 128 channels (eps inside the root), a weight
 *      per channel, and a sigmoid output gate.
 *  [LMSYS-MOVES] same post and section, the three state moves: the
 *      copy-on-write that restores a cached checkpoint into the working slot
 *      and the snapshot at a track boundary are copies on the serial forward
 *      stream; snapshots go to a ping-pong pair whose second slot exists only
 *      around the snapshot; caching donates the latest snapshot's slot index
 *      to the radix tree (no bytes move) and a fresh slot backfills, so a
 *      snapshot never writes a slot a donate handed out.
 *  [B200-CKPT] Kimi K3 B200 deployment notes, the CuTe FlashKDA prefill
 *      item: the prefix cache checkpoints the state every 256 tokens, so
 *      every chunk but a request's last is cut to a multiple of 256 and the
 *      state at a chunk's end is an exact checkpoint.
 *  [B200-DECODE] Kimi K3 B200 deployment notes, the decode items of the
 *      optimisation timeline: a fused KDA decode kernel (conv + KDA + output
 *      norm) for the batch-1 shape, where a decode step is launch-bound.
 *  [LMSYS-SPEC] "SGLang and Miles Add Day-0 Support for Kimi K3", section
 *      "Speculative decoding with DSpark": a per-step planner keeps each
 *      request's verify tokens only while their expected value covers their
 *      cost and trims the rest of the window before the target forward; the
 *      tokens that remain are verified exactly as before.
 *
 * Conventions for every entry point:
 *  - Pointers to tensors are DEVICE pointers unless the name ends in _host.
 *    The caller owns every buffer; the library never allocates device
 *    memory. A plan owns pinned host memory only (see kda_plan_destroy).
 *  - Layouts are row-major (C order); the last dimension is the head
 *    dimension 128. bf16 tensors hold IEEE bfloat16 bit patterns.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream). No call synchronises or reads device memory. Device-data
 *    preconditions (gk <= 0, beta in [0,1], distinct slots, ...) are
 *    documented, not checked; index-like device values (slots, lengths,
 *    ring positions) are clamped or skipped in the kernels so that a bad
 *    value can never address memory outside the buffers described here.
 *  - Every entry point returns a kda_status; kda_last_error() gives a
 *    thread-local message for the last non-OK status. No C++ exception
 *    crosses the ABI. KDA_ERR_DEVICE carries the HIP runtime's error text.
 *  - Two calls in flight must not write the same state, snapshot, output or
 *    ring rows (the single forward stream of [LMSYS-MEM] gives this order),
 *    nor share a prefill workspace (it holds the launch's work counter).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 4
#define KDA_HEAD_DIM 128 /* K = V = 128, fixed at build time */
#define KDA_CHUNK 32     /* prefill chunk length; snap_interval must be a multiple */

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* NULL required pointer, bad count, forbidden alias, bad ring length */
  KDA_ERR_UNSUPPORTED = 2, /* a combination this build does not implement (fp32 inputs with a ring) */
  KDA_ERR_DEVICE = 3,      /* the HIP runtime reported an error while enqueuing work */
  KDA_ERR_HOST_ALLOC = 4,  /* pinned host allocation for a plan failed */
  KDA_ERR_NO_SLOT = 5      /* the state pool has no free slot (nothing was changed) */
} kda_status;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

/* Returns KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

/* Thread-local text for the last non-OK status on this thread ("" if none). */
const char* kda_last_error(void);

/* ---------------------------------------------------------------------------
 * Prefill plan [B200-FKDA]: built once per batch from HOST data and reused by
 * every layer (no device read-back). Work items are (sequence, head, value
 * block) triples; the plan orders them longest sequence first (ties:
 * ascending sequence, then head, then value block), or in input order with
 * KDA_PLAN_FIFO. A value block is a range of the state's value columns: the
 * columns of S evolve independently given the key-side quantities, so a
 * (sequence, head) chain can be split into two halves of 64 columns that run
 * on two workgroups (each recomputes the key side). That doubles the number
 * of chains when there are fewer (sequence, head) pairs than compute units.
 * ------------------------------------------------------------------------- */
typedef struct kda_plan kda_plan;

#define KDA_PLAN_LPT 0  /* longest-processing-time-first (default) */
#define KDA_PLAN_FIFO 1 /* (sequence, head) in input order, for comparison */

/*
 * cu_seqlens_host: int32[n_seq + 1], host memory, non-decreasing, [0] == 0,
 *   last < 2^31. Read before return; the plan keeps its own copy.
 * n_seq >= 1, n_heads >= 1.
 * snap_interval: 0 = no snapshots; else a positive multiple of KDA_CHUNK.
 * order: KDA_PLAN_LPT or KDA_PLAN_FIFO.
 * *out receives an immutable plan, shareable across streams and threads.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_HOST_ALLOC; KDA_ERR_DEVICE if giving back the
 * pinned buffers of destroyed plans failed (kda_host_release; no plan is made).
 */
kda_status kda_plan_create(const int32_t* cu_seqlens_host, int n_seq, int n_heads,
                           int snap_interval, int order, kda_plan** out);

/*
 * kda_plan_create with a choice of value blocks per (sequence, head):
 *   v_blocks = 1: whole 128-column chains (what kda_plan_create builds);
 *   v_blocks = 2: two chains of 64 columns each;
 *   v_blocks = 0: 2 when twice n_seq * n_heads still fits the compute units
 *                 of the current device, else 1 (1 when no device is visible).
 * n_heads <= 65535 (the work list packs head and value block in one int).
 * Results are bitwise the same for every choice.
 * Errors: as kda_plan_create; KDA_ERR_INVALID_ARG for another v_blocks.
 */
kda_status kda_plan_create_ex(const int32_t* cu_seqlens_host, int n_seq, int n_heads,
                              int snap_interval, int order, int v_blocks, kda_plan** out);

/* Value blocks per (sequence, head) of a plan: 1 or 2 (0 for NULL). */
int kda_plan_v_blocks(const kda_plan* plan);

/* Bytes of device workspace a prefill with this plan needs (256 + 16 per item). */
size_t kda_plan_workspace_bytes(const kda_plan* plan);

/* Number of work items (n_seq * n_heads * value blocks). */
int kda_plan_num_items(const kda_plan* plan);

/* Copy the ordered work list to host memory items_host[n_items][4] =
 * (sequence, head | value block << 16, first token, length). For inspection
 * and tests. */
kda_status kda_plan_items(const kda_plan* plan, int32_t* items_host);

/* Enqueue the upload of the work list into `workspace` (device, at least
 * kda_plan_workspace_bytes) and zero its counters. The copy reads the plan's
 * pinned host buffer asynchronously; destroying the plan right after the call
 * is safe (its buffer is only queued for release, see kda_plan_destroy). */
kda_status kda_plan_upload(const kda_plan* plan, void* workspace, void* stream);

/*
 * Free a plan (NULL is a no-op). Makes no HIP runtime call, so it is safe
 * anywhere, including in a garbage collector's finalizer that runs while a
 * graph is being captured: the plan's pinned buffer is queued and given back
 * by the next kda_host_release (which every kda_plan_create calls first).
 * Errors: KDA_ERR_HOST_ALLOC if the queue cannot grow (the buffer is then
 * leaked until the process ends; the plan itself is freed).
 */
kda_status kda_plan_destroy(kda_plan* plan);

/*
 * Free the pinned buffers of destroyed plans (hipHostFree, which waits for
 * the device). Call it outside graph capture; kda_plan_create and
 * kda_plan_create_ex call it before they allocate, and report its failure as
 * theirs. Errors: KDA_ERR_DEVICE with the runtime's text if any free fails
 * (every queued buffer is attempted once and dropped from the queue).
 */
kda_status kda_host_release(void);

/* Inputs of one layer. q, k, v: [rows, H, 128] in the call's q/k/v dtype;
 * gk: fp32 [rows, H, 128], per-token per-key-channel log-decay, gk <= 0;
 * beta: fp32 [rows, H], in [0, 1] (already passed through its sigmoid). */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const float* gk;
  const float* beta;
} kda_inputs;

/* ---------------------------------------------------------------------------
 * Chunked prefill [B200-FKDA], [LMSYS-MEM]. THD-packed batch of the plan's
 * sequences, T = cu_seqlens[n_seq] tokens, H = plan heads.
 *
 *  in        : q, k, v bf16 [T, H, 128]; gk fp32 [T, H, 128]; beta fp32 [T, H].
 *              Any gk <= 0 is exact, -inf (a full reset) included: a 32-token
 *              chunk whose decay summed over it exceeds 60 in some key
 *              channel (where the fast factor form would leave fp32/bf16
 *              range) makes the kernel compute its work item (a sequence's
 *              head, or one value block of it) a second time, in a form with
 *              an exact path for such chunks: that item takes about twice as
 *              long. Range of the state products: the state, and
 *              beta (v - k^T S) of every token, enter fp16 matrix products,
 *              so their entries must stay below 2^15 in magnitude (fp16
 *              overflows at 65504); beyond it o and the states become
 *              non-finite (no error code: nothing is read back). Tested
 *              with state_in ~ N(0, 300^2) and v ~ N(0, 30^2).
 *  state_in  : fp32 [n_seq, H, 128, 128] or NULL (= zeros).
 *  state_out : fp32 [n_seq, H, 128, 128]; may equal state_in (in place);
 *              any other overlap is rejected.
 *  o         : fp32 [T, H, 128]; must not overlap any input or state.
 *  snap      : fp32 [n_seq, snap_slots, H, 128, 128] or NULL. With a plan
 *              snap_interval > 0 and snap != NULL, after the token at
 *              position p (1-based, within its sequence) with
 *              p % snap_interval == 0, the state is copied to slot
 *              (p / snap_interval - 1) % snap_slots (the ping-pong extra
 *              buffer when snap_slots == 2). snap_slots >= 1.
 *  snap_count: int32 [n_seq] or NULL; receives floor(L_n / snap_interval)
 *              (0 without snapshots).
 *  workspace : device scratch of kda_plan_workspace_bytes(plan) bytes. It
 *              holds the work list and a counter that the launch increments
 *              and its last workgroup resets to zero: two prefills in flight
 *              at the same time (on two streams) must use two workspaces,
 *              even with the same plan; calls ordered on one stream may share
 *              one.
 *  scale     : readout scale.
 *  flags     : 0, or KDA_PREFILL_PLAN_RESIDENT when `workspace` already holds
 *              this plan's work list from kda_plan_upload or from an earlier
 *              completed prefill with the same plan and workspace (the
 *              pages' "plan reused by every layer"): the call is then a
 *              single kernel launch. Without the flag the call enqueues the
 *              upload first.
 * Sequences of length 0 get state_out = state_in (or zeros) and no outputs.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_DEVICE.
 */
#define KDA_PREFILL_PLAN_RESIDENT 1
kda_status kda_chunk_prefill(const kda_plan* plan, const kda_inputs* in, const float* state_in,
                             float* state_out, float* o, float* snap, int snap_slots,
                             int32_t* snap_count, void* workspace, float scale, int flags,
                             void* stream);

/*
 * kda_chunk_prefill for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * there is no workspace argument. The plan's work list and its counters go
 * into a static device array inside the library, KDA_NOALLOC_SCRATCH_BYTES
 * long, one per GPU, held until the process ends; each call copies the list
 * there (from the plan's pinned buffer) before its launch. The call makes no
 * allocation (no hipMalloc, hipFree or allocating library routine).
 *  - Every other argument, every precondition and every result as
 *    kda_chunk_prefill with flags = 0; the outputs are bit-identical to it.
 *  - Limit: kda_plan_workspace_bytes(plan) <= KDA_NOALLOC_SCRATCH_BYTES
 *    (65,520 work items); a larger plan is rejected (KDA_ERR_INVALID_ARG).
 *  - All calls on one GPU share the array: two such calls in flight at the
 *    same time on one GPU (on different streams) race. Calls ordered on one
 *    stream are safe (the previous call's contents are overwritten).
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED (device index >= 64),
 * KDA_ERR_DEVICE.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (1 << 20)
kda_status kda_chunk_prefill_noalloc(const kda_plan* plan, const kda_inputs* in, const float* state_in,
                                     float* state_out, float* o, float* snap, int snap_slots,
                                     int32_t* snap_count, float scale, void* stream);

/*
 * Chunked prefill with the output gated RMSNorm fused into its epilogue
 * [B200-NORM]: exactly kda_chunk_prefill, except that instead of o the kernel
 * writes
 *   y[t][h][j] = bf16( o[t][h][j] / sqrt(mean_j' o[t][h][j']^2 + eps)
 *                      * norm_w[j] * sigmoid(gate[t][h][j]) )
 * where o is kda_chunk_prefill's fp32 output (the same bits, never stored),
 * sigmoid(x) = 1 / (1 + e^-x), and bf16 rounding is to nearest even. The
 * arithmetic and its summation order are those of kda_gated_rmsnorm, so y is
 * bit-identical to kda_gated_rmsnorm applied to kda_chunk_prefill's o.
 *
 *  gate   : bf16 [T, H, 128].
 *  norm_w : fp32 [128], one weight per channel, shared by all heads.
 *  eps    : finite, >= 0.
 *  y      : bf16 [T, H, 128]; it may not overlap any input or state buffer.
 *  Every other argument as kda_chunk_prefill. The plan must have one value
 *  block per (sequence, head) (whole rows of o): KDA_ERR_UNSUPPORTED otherwise.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_DEVICE.
 */
kda_status kda_chunk_prefill_gated(const kda_plan* plan, const kda_inputs* in, const void* gate,
                                   const float* norm_w, float eps, const float* state_in,
                                   float* state_out, void* y, float* snap, int snap_slots,
                                   int32_t* snap_count, void* workspace, float scale, int flags,
                                   void* stream);

/*
 * The output gated RMSNorm on its own [B200-NORM], for an o written by
 * kda_chunk_prefill or kda_verify: rows of 128 values,
 *   y[r][j] = bf16( o[r][j] / sqrt(mean_j' o[r][j']^2 + eps) * norm_w[j] * sigmoid(gate[r][j]) ).
 * Fast-math arithmetic (hardware exp2, reciprocal and reciprocal square root)
 * in a fixed summation order: a row is cut into 16 slices of 8 values,
 * slice 4w + q = columns 32w + 4q + {0..3} then 32w + 16 + 4q + {0..3}; each
 * slice's squares are summed in that order, then the slice sums in slice order.
 *
 *  rows   : number of rows (>= 0), e.g. T * H.
 *  o      : fp32 [rows, 128].
 *  gate   : bf16 [rows, 128].
 *  norm_w : fp32 [128].
 *  eps    : finite, >= 0.
 *  y      : bf16 [rows, 128]; may not overlap an input.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_DEVICE.
 */
kda_status kda_gated_rmsnorm(int64_t rows, const float* o, const void* gate, const float* norm_w, float eps,
                             void* y, void* stream);

/*
 * The KDA prologue, the step before the recurrence, in one launch [B200-NORM]
 * (same kernel-fusion items: the three short conv1d calls with their SiLU and
 * the conv-state carry fused, beta's sigmoid fused). For a THD-packed batch of
 * n_seq sequences (token ranges from cu_seqlens), H heads of 128 channels
 * (HC = 128 H per row) and conv width W, for each projection x in (xq, xk, xv):
 *   c_t[ch] = sum_{j < W} conv_w[x][ch][j] * x_{t - W + 1 + j}[ch]
 *             (the W - 1 tokens before a sequence come from conv_state_in)
 *   u_t     = c_t * sigmoid(c_t)                                    (SiLU)
 *   q_t, k_t = u_t / sqrt(sum over the head's 128 channels of u_t^2 + eps)
 *   v_t      = u_t
 * and beta = sigmoid(b_raw), gk = -log(1 + exp(g_raw)). The width and the
 * gate's form are readings (the notes give neither): exp(gk) = sigmoid(-g_raw)
 * is a decay in (0, 1), the input kda_chunk_prefill and kda_verify take.
 *
 *  n_seq, total_tokens, n_heads : N, T, H (H <= 65535, T * H <= 2^33,
 *                   N * 3 * (W - 1) * H * 128 <= 2^38).   conv_width : W in 1..8.
 *  cu_seqlens     : device int32 [N + 1], cu[0] = 0, nondecreasing, cu[N] = T;
 *                   read clamped, so no value of it addresses memory outside
 *                   the buffers here.
 *  xq, xk, xv     : bf16 [T, H, 128].        conv_w : fp32 [3, HC, W].
 *  conv_state_in  : bf16 [N, 3, W - 1, HC] (row W - 2 the latest token) or
 *                   NULL (zeros: fresh sequences).
 *  conv_state_out : same layout, or NULL (not written): the last W - 1 rows of
 *                   each sequence (older state rows for a sequence shorter
 *                   than W - 1). It may not overlap conv_state_in.
 *  b_raw : fp32 [T, H].  g_raw : fp32 [T, H, 128].  eps : finite, >= 0.
 *  q, k, v : bf16 [T, H, 128] (nearest even).  beta : fp32 [T, H].
 *  gk : fp32 [T, H, 128].  No output may overlap an input or another output.
 *  xq, xk, xv, conv_w, conv_state_in/out, g_raw, q, k, v and gk must be 16-byte
 *  aligned.
 * SiLU, sigmoid and the norm's 1/sqrt use the hardware exp2, reciprocal and
 * reciprocal square root (bf16 outputs); gk is accurate to a few fp32 ulps.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_DEVICE.
 */
kda_status kda_prologue(int n_seq, int64_t total_tokens, int n_heads, int conv_width,
                        const int32_t* cu_seqlens, const void* xq, const void* xk, const void* xv,
                        const float* conv_w, const void* conv_state_in, void* conv_state_out,
                        const float* b_raw, const float* g_raw, float eps, void* q, void* k, void* v,
                        float* beta, float* gk, void* stream);

/* ---------------------------------------------------------------------------
 * Per-slot raw-input ring [LMSYS-RSSM], [B200-RING]: for each (slot, layer,
 * head), len entries of (v, k, gk, beta), 1,028 bytes per entry.
 *   k, v : bf16 [n_slots, L, H, len, 128];  gk : fp32 [n_slots, L, H, len, 128];
 *   beta : fp32 [n_slots, L, H, len].  len: a power of two >= 2 * n_tok.
 * Step t of a request with ring start s lives at position (s + t) & (len - 1).
 * ------------------------------------------------------------------------- */
typedef struct {
  void* k;
  void* v;
  float* gk;
  float* beta;
  int len;
} kda_ring;

/*
 * Speculative multi-token verify of one layer [LMSYS-RSSM]: one launch per
 * layer; reads the committed state and never writes it.
 *
 *  batch, n_tok        : requests and draft tokens per request (gamma + 1).
 *  n_heads, n_layers   : H and L of the pools; layer in [0, L).
 *  n_slots             : first dimension of the pools and the ring.
 *  qkv_dtype           : KDA_BF16, or KDA_F32 (only with ring == NULL).
 *  in                  : rows b * n_tok + t of [batch * n_tok, H, 128].
 *  state_pool          : fp32 [n_slots, L, H, 128, 128], read only.
 *  slot_idx            : int32 [batch], distinct; a slot outside [0, n_slots)
 *                        makes the kernel skip that request.
 *  o                   : fp32 [batch * n_tok, H, 128].
 *  ring, ring_start    : ring may be NULL (nothing recorded); ring_start int32
 *                        [batch] or NULL (= 0).
 *  commit_len          : int32 [batch] or NULL. For request b with
 *                        c = min(commit_len[b], n_tok) > 0, the state after c
 *                        steps is written to commit_pool[slot_b, layer, h]
 *                        (the recurrent commit; a decode step is n_tok = 1,
 *                        commit_len = 1, commit_pool = state_pool).
 *  commit_pool         : like state_pool, or NULL; may equal state_pool, may
 *                        not overlap it otherwise.
 * Arithmetic: with bf16 inputs, n_tok <= 16 and no commit, the window is one
 * chunk of the chunked form on the matrix cores (the served path); otherwise
 * the token-by-token recurrence (whose commit kda_replay_fold reproduces bit
 * for bit). Both are exact for any gk <= 0 (-inf included): a window whose
 * decay summed over it exceeds 80 in some key channel forms its intra-window
 * products pairwise. On the chunked path the committed state and
 * beta (v - k^T S0) enter fp16 products: their entries must stay below 2^15.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_DEVICE.
 */
kda_status kda_verify(int batch, int n_tok, int n_heads, int n_layers, int layer, int n_slots,
                      kda_dtype qkv_dtype, const kda_inputs* in, const float* state_pool,
                      const int32_t* slot_idx, float* o, const kda_ring* ring,
                      const int32_t* ring_start, const int32_t* commit_len, float* commit_pool,
                      float scale, void* stream);

/*
 * Replay fold [LMSYS-RSSM]: one launch over every (request, layer, head).
 * Advances state_pool[slot_b, l, h] in place by the first accepted_len[b]
 * ring entries (from ring_start[b]) with the same step and reduction order
 * as kda_verify, so the result is bit-identical to kda_verify's commit after
 * that many steps. Entries past the accepted prefix are never read.
 *
 *  accepted_len : int32 [batch]; 0 leaves the state untouched; values are
 *                 clamped to [0, ring->len / 2].
 *  slot_idx, ring_start : as for kda_verify.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_DEVICE.
 */
kda_status kda_replay_fold(int batch, int n_heads, int n_layers, int n_slots, float* state_pool,
                           const int32_t* slot_idx, const kda_ring* ring,
                           const int32_t* ring_start, const int32_t* accepted_len, void* stream);

/*
 * Fused fold-then-verify of one layer [LMSYS-RSSM]. The fold of a speculative
 * step and the verify of the next step read the same committed state; this
 * entry point does both in one pass over it. For each request b and head h of
 * `layer`:
 *   1. fold: advance state_pool[slot_b, layer, h] in place by the first
 *      fold_len[b] ring entries from position fold_start[b], exactly as
 *      kda_replay_fold does (same step function, lane ownership and reduction
 *      order: the state is bit-identical to kda_replay_fold's);
 *   2. verify: from that state, exactly as kda_verify without a commit (o and
 *      the ring entries at ring_start[b] + t are bit-identical to kda_verify's
 *      on the folded pool).
 * So a step sequence "verify; fold over all layers" becomes one
 * kda_fold_verify per layer per step, folding the previous step's window.
 *
 *  batch .. slot_idx, o : as kda_verify; bf16 q/k/v only, 1 <= n_tok <= 8.
 *  ring                 : required, ring->len a power of two in [2 n_tok, 16]
 *                         (so at most 8 entries are folded).
 *  fold_start           : int32 [batch] or NULL (= 0): ring position of the
 *                         previous window's first entry.
 *  fold_len             : int32 [batch], required; 0 folds nothing (the state
 *                         is not written); clamped to [0, ring->len / 2].
 *  ring_start           : int32 [batch] or NULL (= 0): where this step's
 *                         entries go. Precondition (not checked): the folded
 *                         entries and this step's entries do not overlap
 *                         modulo ring->len (a ring of at least 2 n_tok holds
 *                         the window being folded plus the next one).
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_DEVICE.
 */
kda_status kda_fold_verify(int batch, int n_tok, int n_heads, int n_layers, int layer, int n_slots,
                           const kda_inputs* in, float* state_pool, const int32_t* slot_idx, float* o,
                           const kda_ring* ring, const int32_t* fold_start, const int32_t* fold_len,
                           const int32_t* ring_start, float scale, void* stream);

/*
 * Ragged verify of one layer [LMSYS-SPEC], [B200-RING]: request b verifies
 * its own trimmed window of n_b draft tokens, packed back to back. Each
 * window is verified exactly as kda_verify without a commit verifies a
 * window of that length (o and the ring entries are bit-identical to a
 * kda_verify call with n_tok = n_b for that request); the committed state is
 * never written. A later kda_replay_fold may fold up to n_b of the recorded
 * entries.
 *
 *  batch          : requests (>= 0).
 *  max_tok        : 1..16, a bound on every n_b (windows longer are cut).
 *  total_tok      : rows of the packed tensors (>= 0; 0 = nothing to do).
 *  n_heads .. n_slots, state_pool, slot_idx : as kda_verify.
 *  in             : bf16 q/k/v, fp32 gk/beta; row cu_tok[b] + t of
 *                   [total_tok, H, 128] is token t of request b.
 *  cu_tok         : int32 [batch + 1], required: the windows' prefix sums,
 *                   cu_tok[0] = 0, nondecreasing, cu_tok[batch] = total_tok.
 *                   Read on the device and clamped there: the window of b
 *                   is rows [s, e) with s = cu_tok[b] and e = cu_tok[b + 1]
 *                   clamped into [0, total_tok] and e >= s, cut to max_tok
 *                   rows; so no value of cu_tok addresses a row outside the
 *                   tensors. An empty window writes nothing.
 *  o              : fp32 [total_tok, H, 128]; rows of a skipped request
 *                   (invalid slot) are not written.
 *  ring, ring_start : as kda_verify; ring->len >= 2 * max_tok. Entry t < n_b
 *                   of request b goes to (ring_start[b] + t) & (len - 1);
 *                   the other entries of the ring are not touched.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_DEVICE.
 */
kda_status kda_verify_ragged(int batch, int max_tok, int total_tok, int n_heads, int n_layers, int layer,
                             int n_slots, const kda_inputs* in, const int32_t* cu_tok,
                             const float* state_pool, const int32_t* slot_idx, float* o,
                             const kda_ring* ring, const int32_t* ring_start, float scale, void* stream);

/*
 * One decode step of a KDA layer in one launch [B200-DECODE]: for each request
 * b (one new token) and head h, the prologue of kda_prologue for that token
 * (short conv with the conv state, SiLU, q/k L2 norm with qk_eps, beta and
 * gk), the recurrent step of kda_verify with n_tok = 1 and the commit written
 * in place into state_pool, and the output gated RMSNorm of kda_gated_rmsnorm
 * with norm_eps. y, the committed state and the conv state are bit for bit
 * those of kda_prologue, kda_verify (commit_len = 1, commit_pool = state_pool)
 * and kda_gated_rmsnorm run one after another.
 *  batch, n_heads (<= 65535), n_layers, layer, n_slots : as kda_verify.
 *  conv_width : W in 1..8.
 *  xq, xk, xv : bf16 [batch, H, 128], the token's projections.
 *  conv_w     : fp32 [3, H * 128, W].
 *  conv_state : bf16 [batch, 3, W - 1, H * 128] (row W - 2 the newest),
 *               updated in place (the token becomes the newest row); NULL
 *               only when W = 1.
 *  b_raw : fp32 [batch, H].  g_raw : fp32 [batch, H, 128].
 *  state_pool : fp32 [n_slots, L, H, 128, 128], updated in place.
 *  slot_idx   : device int32 [batch]; a slot outside [0, n_slots) skips the
 *               request whole (its outputs and conv state are not written).
 *  gate : bf16 [batch, H, 128].  norm_w : fp32 [128].
 *  y : bf16 [batch, H, 128].  o : fp32 [batch, H, 128] (the step's output
 *      before the norm) or NULL.
 *  Row buffers 16-byte aligned; no output may overlap an input or another
 *  output; distinct slots.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_DEVICE.
 */
kda_status kda_decode(int batch, int n_heads, int n_layers, int layer, int n_slots, int conv_width,
                      const void* xq, const void* xk, const void* xv, const float* conv_w, void* conv_state,
                      const float* b_raw, const float* g_raw, float* state_pool, const int32_t* slot_idx,
                      const void* gate, const float* norm_w, float qk_eps, float norm_eps, float scale, void* y,
                      float* o, void* stream);

/* ---------------------------------------------------------------------------
 * Prefix-cache state moves [LMSYS-MOVES] [B200-CKPT]. The state pool is the
 * one kda_verify and kda_replay_fold take: fp32 [n_slots, n_layers, H, 128,
 * 128], a slot holding every layer and head of one request. A request's live
 * state is its working slot. Restores and snapshots are whole-slot copies
 * (kda_state_move) enqueued on the forward stream between the forwards that
 * produce and consume the state; donating moves ownership only.
 * ------------------------------------------------------------------------- */

/* One whole-slot copy: pool[dst] = pool[src]. */
typedef struct {
  int32_t src;
  int32_t dst;
} kda_move;

/*
 * Copies pool[moves[i].src] to pool[moves[i].dst] for i < n_moves, bit for
 * bit, in one launch [LMSYS-MOVES].
 *  n_moves     : >= 0.   moves : DEVICE kda_move[n_moves].
 *  n_slots     : slots in the pool (>= 1).
 *  slot_floats : floats per slot (n_layers * H * 128 * 128), a positive
 *                multiple of 4.
 *  pool        : DEVICE fp32 [n_slots, slot_floats], 16-byte aligned.
 * A move with src or dst outside [0, n_slots), or src == dst, is skipped.
 * No move may write a slot another move of the same call reads or writes
 * (the slot protocol below never emits such a pair); moves of separate calls
 * are ordered by the stream.
 * Errors: KDA_ERR_INVALID_ARG, KDA_ERR_DEVICE.
 */
kda_status kda_state_move(int n_moves, const kda_move* moves, int n_slots, int64_t slot_floats, float* pool,
                          void* stream);

/*
 * Checkpoint-aligned chunking [B200-CKPT], host only. Splits an extend of
 * len tokens that starts after pos0 tokens already in the state into chunks
 * of at most budget tokens. Every chunk but the last ends at the last
 * multiple of align within its budget (an exact checkpoint position); where
 * no multiple of align lies within the budget the chunk takes the whole
 * budget. The last chunk takes the rest (<= budget).
 *  pos0 >= 0, len >= 0, budget >= 1, align >= 1 (256 for the cache).
 *  lens_host : host int64[max_chunks] receiving the chunk lengths.
 *  *n_chunks : the number of chunks (also when it exceeds max_chunks, which
 *              returns KDA_ERR_INVALID_ARG; lens_host then holds the first
 *              max_chunks).
 * Errors: KDA_ERR_INVALID_ARG.
 */
kda_status kda_chunk_split(int64_t pos0, int64_t len, int64_t budget, int64_t align, int64_t* lens_host,
                           int max_chunks, int* n_chunks);

/*
 * Slot ownership under the three moves [LMSYS-MOVES], host only. Every slot
 * of the pool has one owner: the free list, one open request, or the tree
 * (the prefix cache). The calls change owners and fill in the copies to
 * enqueue with kda_state_move; they never touch device memory and are not
 * thread-safe (one scheduler thread owns a kda_slots).
 *   open     : takes a free slot as the working slot; with cached_slot (a
 *              slot the tree owns) also returns the copy-on-write move
 *              cached_slot -> working (the tree's checkpoint is not changed).
 *   snapshot : takes a free slot as the target (the ping-pong pair's second
 *              slot), returns the move working -> target, makes the target
 *              the latest snapshot and frees the one it supersedes (later
 *              writes to that slot are ordered after this copy by the
 *              stream).
 *   donate   : hands the latest snapshot to the tree (no copy); the next
 *              snapshot takes a fresh slot, so a snapshot never writes a slot
 *              the tree owns.
 *   close    : frees the working slot and a snapshot not donated.
 *   release  : the tree evicts a slot it owns back to the free list.
 * A request holds at most two slots between calls (working and latest).
 * KDA_ERR_NO_SLOT leaves every owner unchanged. KDA_ERR_INVALID_ARG covers a
 * restore from a slot the tree does not own, a request this pool did not
 * open (or already closed), a donate without a snapshot, and a release of a
 * slot the tree does not own.
 */
typedef struct kda_slots kda_slots;

typedef struct {
  int32_t id;      /* request id, >= 0 while open; -1 after close */
  int32_t working; /* the slot every forward reads and overwrites */
  int32_t snap;    /* the latest snapshot's slot, -1 = none */
} kda_request_slots;

#define KDA_SLOT_FREE (-1) /* kda_slots_owner: on the free list */
#define KDA_SLOT_TREE (-2) /* kda_slots_owner: owned by the tree */

kda_status kda_slots_create(int n_slots, kda_slots** out);
void kda_slots_destroy(kda_slots* slots);
int kda_slots_free_count(const kda_slots* slots);
/* The owner of a slot: a request id, KDA_SLOT_FREE or KDA_SLOT_TREE; -3 for a bad slot. */
int kda_slots_owner(const kda_slots* slots, int32_t slot);
/* restore_host: host kda_move[1], required when cached_slot != -1; *n_moves = 0 or 1. */
kda_status kda_request_open(kda_slots* slots, int32_t cached_slot, kda_request_slots* r, kda_move* restore_host,
                            int* n_moves);
kda_status kda_request_snapshot(kda_slots* slots, kda_request_slots* r, kda_move* move_host);
kda_status kda_request_donate(kda_slots* slots, kda_request_slots* r, int32_t* slot);
kda_status kda_request_close(kda_slots* slots, kda_request_slots* r);
kda_status kda_slot_release(kda_slots* slots, int32_t slot);

/* -------------------------------------------------------------------------
 * Measurement probes (diagnostics, not part of the method). The rates the
 * chip reaches on the simplest work -- a streaming copy, a streaming read and
 * a loop of independent bf16 matrix-core products -- so that a benchmark can
 * report its kernels against what this GPU attains in the same run beside the
 * vendor peaks. Asynchronous on stream; they read or write only the buffers
 * named. Errors: KDA_ERR_INVALID_ARG, KDA_ERR_DEVICE.
 * ------------------------------------------------------------------------- */

/* dst = src, bytes each (a positive multiple of 16), both DEVICE, 16-byte
 * aligned, not overlapping. Moves 2 * bytes through HBM. */
kda_status kda_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Reads bytes (a positive multiple of 16) of DEVICE src (16-byte aligned)
 * once and writes one partial sum per thread to DEVICE sink (sink_floats >=
 * 256; the grid is at most sink_floats / 256 workgroups of 256 threads). */
kda_status kda_probe_read(const void* src, int64_t bytes, float* sink, int64_t sink_floats, void* stream);

/* Runs iters (1 .. 2^30, rounded up to a multiple of 32) rounds of eight
 * independent 16x16x32 bf16 MFMAs per wave (operands derived from seed and
 * the lane) and writes one sum per thread to
 * DEVICE sink (sink_floats >= 256). *flop (HOST) receives the flops the
 * launch performs. */
kda_status kda_probe_mfma(int iters, float seed, float* sink, int64_t sink_floats, int64_t* flop, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
