// kda_api.cpp -- host side of libkda: argument validation, the prefill plan
// (longest-first work list built from host data), and the kernel launches.
// See include/kda.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local std::string g_err;

kda_status fail(kda_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

kda_status ok() { return KDA_OK; }

}  // namespace

kda_status kda::fail(kda_status s, const char* msg) { return ::fail(s, msg); }

namespace {

kda_status device_fail(const char* what, hipError_t e) {
  return fail(KDA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

// [a, a + na) and [b, b + nb) share a byte
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

constexpr size_t kState = (size_t)KDA_HEAD_DIM * KDA_HEAD_DIM * sizeof(float);

}  // namespace

namespace {

// Pinned work-list buffers of destroyed plans. kda_plan_destroy makes no HIP
// runtime call (it may run from a garbage collector's finalizer, at any
// moment, including while another thread or the same one captures a graph,
// where a synchronising call such as hipHostFree would invalidate the
// capture); it queues the buffer here and kda_host_release frees it later.
std::mutex g_released_mu;
std::vector<void*> g_released;

}  // namespace

struct kda_plan {
  int n_seq = 0, n_heads = 0, snap_interval = 0, order = 0, v_blocks = 1, n_items = 0;
  int64_t total_tokens = 0;
  std::vector<int32_t> items;  // host copy, 4 ints per item
  void* upload = nullptr;      // header + items, pinned when the runtime allows
  bool pinned = false;
  size_t bytes = 0;
};

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_last_error(void) { return g_err.c_str(); }

kda_status kda_plan_create(const int32_t* cu_seqlens_host, int n_seq, int n_heads, int snap_interval,
                           int order, kda_plan** out) {
  return kda_plan_create_ex(cu_seqlens_host, n_seq, n_heads, snap_interval, order, 1, out);
}

kda_status kda_host_release(void) {
  std::vector<void*> bufs;
  {
    std::lock_guard<std::mutex> lock(g_released_mu);
    bufs.swap(g_released);
  }
  std::string err;
  size_t failed = 0;
  for (void* b : bufs) {
    const hipError_t e = hipHostFree(b);
    if (e != hipSuccess) {
      if (failed++ == 0) err = hipGetErrorString(e);
    }
  }
  if (failed)
    return fail(KDA_ERR_DEVICE, "kda_host_release: hipHostFree failed for " + std::to_string(failed) + " of " +
                                    std::to_string(bufs.size()) + " buffers: " + err);
  return ok();
}

kda_status kda_plan_create_ex(const int32_t* cu_seqlens_host, int n_seq, int n_heads, int snap_interval,
                              int order, int v_blocks, kda_plan** out) {
  if (!out) return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: out is NULL");
  *out = nullptr;
  {
    // creating a plan allocates pinned memory (not allowed under capture either), so it is
    // also where the buffers of destroyed plans are given back
    const kda_status rs = kda_host_release();
    if (rs != KDA_OK) return fail(rs, std::string("kda_plan_create: ") + kda_last_error());
  }
  if (!cu_seqlens_host) return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: cu_seqlens_host is NULL");
  if (n_seq < 1 || n_heads < 1) return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: n_seq and n_heads must be >= 1");
  if (n_heads > 0xffff) return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: n_heads must be <= 65535");
  if (v_blocks < 0 || v_blocks > 2) return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: v_blocks must be 0, 1 or 2");
  if (v_blocks == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        2LL * n_seq * n_heads <= cus)
      v_blocks = 2;
    else
      v_blocks = 1;
    (void)hipGetLastError();  // no device visible: the choice falls back to 1
  }
  if ((int64_t)n_seq * n_heads * v_blocks > 0x7fffffffLL) return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: too many work items");
  if (snap_interval < 0 || snap_interval % KDA_CHUNK != 0)
    return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: snap_interval must be 0 or a positive multiple of KDA_CHUNK (32)");
  if (order != KDA_PLAN_LPT && order != KDA_PLAN_FIFO) return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: bad order");
  if (cu_seqlens_host[0] != 0) return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: cu_seqlens[0] must be 0");
  for (int n = 0; n < n_seq; ++n)
    if (cu_seqlens_host[n + 1] < cu_seqlens_host[n])
      return fail(KDA_ERR_INVALID_ARG, "kda_plan_create: cu_seqlens must be non-decreasing");

  kda_plan* p = new (std::nothrow) kda_plan;
  if (!p) return fail(KDA_ERR_HOST_ALLOC, "kda_plan_create: out of host memory");
  p->n_seq = n_seq;
  p->n_heads = n_heads;
  p->snap_interval = snap_interval;
  p->order = order;
  p->v_blocks = v_blocks;
  p->n_items = n_seq * n_heads * v_blocks;
  p->total_tokens = cu_seqlens_host[n_seq];
  const int per_seq = n_heads * v_blocks;
  std::vector<int> idx(p->n_items);
  for (int i = 0; i < p->n_items; ++i) idx[i] = i;  // item i = (n = i / (H vb), h, value block)
  if (order == KDA_PLAN_LPT) {
    // longest sequence first; equal lengths keep (sequence, head, value block) ascending
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) {
      const int na = a / per_seq, nb = b / per_seq;
      return (cu_seqlens_host[na + 1] - cu_seqlens_host[na]) > (cu_seqlens_host[nb + 1] - cu_seqlens_host[nb]);
    });
  }
  p->items.resize((size_t)p->n_items * 4);
  for (int i = 0; i < p->n_items; ++i) {
    const int n = idx[i] / per_seq, h = (idx[i] % per_seq) / v_blocks, vb = idx[i] % v_blocks;
    p->items[4 * i + 0] = n;
    p->items[4 * i + 1] = h | (vb << 16);
    p->items[4 * i + 2] = cu_seqlens_host[n];
    p->items[4 * i + 3] = cu_seqlens_host[n + 1] - cu_seqlens_host[n];
  }
  p->bytes = sizeof(kda::PrefillWsHeader) + p->items.size() * sizeof(int32_t);
  if (hipHostMalloc(&p->upload, p->bytes, hipHostMallocDefault) == hipSuccess) {
    p->pinned = true;
  } else {
    (void)hipGetLastError();  // no device here: keep a pageable copy for inspection
    p->upload = std::malloc(p->bytes);
    if (!p->upload) {
      delete p;
      return fail(KDA_ERR_HOST_ALLOC, "kda_plan_create: out of host memory");
    }
  }
  std::memset(p->upload, 0, sizeof(kda::PrefillWsHeader));
  std::memcpy(static_cast<char*>(p->upload) + sizeof(kda::PrefillWsHeader), p->items.data(),
              p->items.size() * sizeof(int32_t));
  *out = p;
  return ok();
}

size_t kda_plan_workspace_bytes(const kda_plan* p) { return p ? p->bytes : 0; }

int kda_plan_num_items(const kda_plan* p) { return p ? p->n_items : 0; }

int kda_plan_v_blocks(const kda_plan* p) { return p ? p->v_blocks : 0; }

kda_status kda_plan_items(const kda_plan* p, int32_t* items_host) {
  if (!p || !items_host) return fail(KDA_ERR_INVALID_ARG, "kda_plan_items: NULL argument");
  std::memcpy(items_host, p->items.data(), p->items.size() * sizeof(int32_t));
  return ok();
}

kda_status kda_plan_upload(const kda_plan* p, void* workspace, void* stream) {
  if (!p || !workspace) return fail(KDA_ERR_INVALID_ARG, "kda_plan_upload: NULL argument");
  const hipError_t e = hipMemcpyAsync(workspace, p->upload, p->bytes, hipMemcpyHostToDevice,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_plan_upload", e);
  return ok();
}

kda_status kda_plan_destroy(kda_plan* p) {
  if (!p) return ok();
  if (p->pinned) {
    std::lock_guard<std::mutex> lock(g_released_mu);
    try {
      g_released.push_back(p->upload);  // freed by the next kda_host_release (no HIP call here)
    } catch (...) {
      // the queue could not grow: the buffer stays allocated until the process ends
      delete p;
      return fail(KDA_ERR_HOST_ALLOC, "kda_plan_destroy: no host memory to queue the pinned buffer (leaked)");
    }
  } else {
    std::free(p->upload);
  }
  delete p;
  return ok();
}

// kda_chunk_prefill and kda_chunk_prefill_gated: the same checks and launch; the gated form writes
// bf16 y (the output gated RMSNorm of o) instead of fp32 o
static kda_status prefill_call(const char* fn, const kda_plan* p, const kda_inputs* in, const float* state_in,
                               float* state_out, float* o, const void* gate, const float* norm_w, float eps, void* y,
                               float* snap, int snap_slots, int32_t* snap_count, void* workspace, float scale,
                               int flags, void* stream) {
  const bool gated = y != nullptr;
  auto bad = [&](kda_status st, const char* what) { return fail(st, std::string(fn) + ": " + what); };
  if (!p) return bad(KDA_ERR_INVALID_ARG, "plan is NULL");
  if (!in) return bad(KDA_ERR_INVALID_ARG, "inputs are NULL");
  if (!state_out) return bad(KDA_ERR_INVALID_ARG, "state_out is NULL");
  if (!workspace) return bad(KDA_ERR_INVALID_ARG, "workspace is NULL");
  if (flags & ~KDA_PREFILL_PLAN_RESIDENT) return bad(KDA_ERR_INVALID_ARG, "unknown flags");
  if (gated && !(eps >= 0.f && eps < INFINITY)) return bad(KDA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (gated && p->v_blocks != 1)
    return bad(KDA_ERR_UNSUPPORTED, "the fused norm needs whole rows: a plan with one value block per (sequence, head)");
  const int64_t T = p->total_tokens;
  const int H = p->n_heads;
  void* out = gated ? y : static_cast<void*>(o);
  if (T > 0 && (!in->q || !in->k || !in->v || !in->gk || !in->beta || !out))
    return bad(KDA_ERR_INVALID_ARG, gated ? "q, k, v, gk, beta and y are required" : "q, k, v, gk, beta and o are required");
  if (gated && T > 0 && (!gate || !norm_w)) return bad(KDA_ERR_INVALID_ARG, "gate and norm_w are required");
  const bool snaps = p->snap_interval > 0 && snap != nullptr;
  if (snaps && snap_slots < 1) return bad(KDA_ERR_INVALID_ARG, "snap_slots must be >= 1");
  const size_t tok = (size_t)T * H;
  const size_t qkv_b = tok * KDA_HEAD_DIM * 2, gk_b = tok * KDA_HEAD_DIM * 4, beta_b = tok * 4;
  const size_t o_b = tok * KDA_HEAD_DIM * (gated ? 2 : 4);
  const size_t st_b = (size_t)p->n_seq * H * kState;
  const size_t snap_b = snaps ? (size_t)p->n_seq * snap_slots * H * kState : 0;
  const void* ins[7] = {in->q, in->k, in->v, in->gk, in->beta, gated ? gate : nullptr, gated ? norm_w : nullptr};
  const size_t insz[7] = {qkv_b, qkv_b, qkv_b, gk_b, beta_b, qkv_b, (size_t)KDA_HEAD_DIM * 4};
  for (int i = 0; i < 7; ++i) {
    if (overlap(out, o_b, ins[i], insz[i])) return bad(KDA_ERR_INVALID_ARG, gated ? "y overlaps an input" : "o overlaps an input");
    if (overlap(state_out, st_b, ins[i], insz[i])) return bad(KDA_ERR_INVALID_ARG, "state_out overlaps an input");
    if (snaps && overlap(snap, snap_b, ins[i], insz[i])) return bad(KDA_ERR_INVALID_ARG, "snap overlaps an input");
  }
  if (overlap(out, o_b, state_out, st_b) || overlap(out, o_b, state_in, st_b) || (snaps && overlap(out, o_b, snap, snap_b)))
    return bad(KDA_ERR_INVALID_ARG, gated ? "y overlaps a state buffer" : "o overlaps a state buffer");
  if (state_in != state_out && overlap(state_in, st_b, state_out, st_b))
    return bad(KDA_ERR_INVALID_ARG, "state_in and state_out overlap without being equal");
  if (snaps && (overlap(snap, snap_b, state_out, st_b) || overlap(snap, snap_b, state_in, st_b)))
    return bad(KDA_ERR_INVALID_ARG, "snap overlaps a state buffer");
  if (overlap(workspace, p->bytes, out, o_b) || overlap(workspace, p->bytes, state_out, st_b))
    return bad(KDA_ERR_INVALID_ARG, "workspace overlaps an output");

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!(flags & KDA_PREFILL_PLAN_RESIDENT)) {
    const kda_status st = kda_plan_upload(p, workspace, stream);
    if (st != KDA_OK) return st;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(fn, e);
  kda::PrefillArgs a{};
  a.n_seq = p->n_seq;
  a.n_heads = H;
  a.n_items = p->n_items;
  a.total_tokens = T;
  a.q = static_cast<const uint16_t*>(in->q);
  a.k = static_cast<const uint16_t*>(in->k);
  a.v = static_cast<const uint16_t*>(in->v);
  a.gk = in->gk;
  a.beta = in->beta;
  a.state_in = state_in;
  a.state_out = state_out;
  a.o = gated ? nullptr : o;
  a.snap = snaps ? snap : nullptr;
  a.snap_slots = snaps ? snap_slots : 0;
  a.snap_interval = snaps ? p->snap_interval : 0;
  a.snap_count = snap_count;
  a.ws = static_cast<kda::PrefillWsHeader*>(workspace);
  a.items = reinterpret_cast<const int4*>(static_cast<char*>(workspace) + sizeof(kda::PrefillWsHeader));
  a.n_vblk = p->v_blocks;
  a.scale = scale;
  if (gated) {
    a.gate = static_cast<const uint16_t*>(gate);
    a.norm_w = norm_w;
    a.eps = eps;
    a.y = static_cast<uint16_t*>(y);
  }
  const int grid = std::min(p->n_items, kda::prefill_max_grid(dev));
  e = kda::launch_prefill(a, grid, s);
  if (e != hipSuccess) return device_fail(fn, e);
  return ok();
}

kda_status kda_chunk_prefill(const kda_plan* p, const kda_inputs* in, const float* state_in, float* state_out,
                             float* o, float* snap, int snap_slots, int32_t* snap_count, void* workspace,
                             float scale, int flags, void* stream) {
  return prefill_call("kda_chunk_prefill", p, in, state_in, state_out, o, nullptr, nullptr, 0.f, nullptr, snap,
                      snap_slots, snap_count, workspace, scale, flags, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The prefill without a caller workspace: the work list and its counters live in
// `scratch`, a static device array of this library (one copy per GPU, kept until
// the process ends). Host code never passes `scratch` itself to a kernel or a copy:
// its name is a host-side stand-in. The device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the calling thread's current device and that device's address of `scratch`
kda_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail("kda_chunk_prefill_noalloc: hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_prefill_noalloc: device index >= 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_fail("kda_chunk_prefill_noalloc: hipGetSymbolAddress(scratch)", e);
    if (!ptr) return fail(KDA_ERR_DEVICE, "kda_chunk_prefill_noalloc: hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

extern "C" {

kda_status kda_chunk_prefill_noalloc(const kda_plan* p, const kda_inputs* in, const float* state_in,
                                     float* state_out, float* o, float* snap, int snap_slots, int32_t* snap_count,
                                     float scale, void* stream) {
  if (!p) return fail(KDA_ERR_INVALID_ARG, "kda_chunk_prefill_noalloc: plan is NULL");
  if (kda_plan_workspace_bytes(p) > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
    return fail(KDA_ERR_INVALID_ARG, "kda_chunk_prefill_noalloc: the plan's work list (" +
                                         std::to_string(kda_plan_workspace_bytes(p)) + " bytes) exceeds the " +
                                         std::to_string(KDA_NOALLOC_SCRATCH_BYTES) + "-byte static scratch");
  void* ws = nullptr;
  const kda_status st = scratch_ptr(&ws);
  if (st != KDA_OK) return st;
  // the upload rewrites the whole list and zeroes the counters, so a previous call's contents never matter
  return prefill_call("kda_chunk_prefill_noalloc", p, in, state_in, state_out, o, nullptr, nullptr, 0.f, nullptr, snap,
                      snap_slots, snap_count, ws, scale, 0, stream);
}

kda_status kda_chunk_prefill_gated(const kda_plan* p, const kda_inputs* in, const void* gate, const float* norm_w,
                                   float eps, const float* state_in, float* state_out, void* y, float* snap,
                                   int snap_slots, int32_t* snap_count, void* workspace, float scale, int flags,
                                   void* stream) {
  if (!y) return fail(KDA_ERR_INVALID_ARG, "kda_chunk_prefill_gated: y is NULL");
  return prefill_call("kda_chunk_prefill_gated", p, in, state_in, state_out, nullptr, gate, norm_w, eps, y, snap,
                      snap_slots, snap_count, workspace, scale, flags, stream);
}

kda_status kda_gated_rmsnorm(int64_t rows, const float* o, const void* gate, const float* norm_w, float eps, void* y,
                             void* stream) {
  if (rows < 0) return fail(KDA_ERR_INVALID_ARG, "kda_gated_rmsnorm: rows < 0");
  if (!(eps >= 0.f && eps < INFINITY)) return fail(KDA_ERR_INVALID_ARG, "kda_gated_rmsnorm: eps must be finite and >= 0");
  if (rows == 0) return ok();
  if (rows > ((int64_t)1 << 34)) return fail(KDA_ERR_INVALID_ARG, "kda_gated_rmsnorm: too many rows");
  if (!o || !gate || !norm_w || !y) return fail(KDA_ERR_INVALID_ARG, "kda_gated_rmsnorm: o, gate, norm_w and y are required");
  const size_t yb = (size_t)rows * KDA_HEAD_DIM * 2;
  if (overlap(y, yb, o, (size_t)rows * KDA_HEAD_DIM * 4) || overlap(y, yb, gate, yb) ||
      overlap(y, yb, norm_w, (size_t)KDA_HEAD_DIM * 4))
    return fail(KDA_ERR_INVALID_ARG, "kda_gated_rmsnorm: y overlaps an input");
  const hipError_t e = kda::launch_gated_rmsnorm(rows, o, static_cast<const uint16_t*>(gate), norm_w, eps,
                                                 static_cast<uint16_t*>(y), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_gated_rmsnorm: launch", e);
  return ok();
}

kda_status kda_fold_verify(int batch, int n_tok, int n_heads, int n_layers, int layer, int n_slots,
                           const kda_inputs* in, float* state_pool, const int32_t* slot_idx, float* o,
                           const kda_ring* ring, const int32_t* fold_start, const int32_t* fold_len,
                           const int32_t* ring_start, float scale, void* stream) {
  if (batch < 0 || n_tok < 1 || n_heads < 1 || n_layers < 1 || n_slots < 1 || layer < 0 || layer >= n_layers)
    return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: bad batch/n_tok/n_heads/n_layers/layer/n_slots");
  if (n_tok > 8) return fail(KDA_ERR_UNSUPPORTED, "kda_fold_verify: n_tok must be <= 8");
  if ((int64_t)batch * n_heads > 0x7fffffffLL) return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: grid too large");
  if (!ring || !ring->k || !ring->v || !ring->gk || !ring->beta)
    return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: the ring is required");
  if (!pow2(ring->len) || ring->len < 2 * n_tok)
    return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: ring length must be a power of two >= 2 * n_tok");
  if (ring->len > 16) return fail(KDA_ERR_UNSUPPORTED, "kda_fold_verify: ring length must be <= 16");
  if (!fold_len) return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: fold_len is required");
  if (batch == 0) return ok();
  if (!in || !in->q || !in->k || !in->v || !in->gk || !in->beta)
    return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: q, k, v, gk and beta are required");
  if (!state_pool || !slot_idx || !o)
    return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: state_pool, slot_idx and o are required");
  const size_t rows = (size_t)batch * n_tok * n_heads;
  const size_t pool_b = (size_t)n_slots * n_layers * n_heads * kState;
  const size_t o_b = rows * KDA_HEAD_DIM * 4;
  const size_t ring_units = (size_t)n_slots * n_layers * n_heads * ring->len;
  const void* bufs[] = {in->q, in->k, in->v, in->gk, in->beta, state_pool};
  const size_t bsz[] = {rows * KDA_HEAD_DIM * 2, rows * KDA_HEAD_DIM * 2, rows * KDA_HEAD_DIM * 2,
                        rows * KDA_HEAD_DIM * 4, rows * 4, pool_b};
  const void* rb[] = {ring->k, ring->v, ring->gk, ring->beta};
  const size_t rs[] = {ring_units * KDA_HEAD_DIM * 2, ring_units * KDA_HEAD_DIM * 2, ring_units * KDA_HEAD_DIM * 4,
                       ring_units * 4};
  for (int i = 0; i < 6; ++i) {
    if (overlap(o, o_b, bufs[i], bsz[i])) return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: o overlaps an input or the pool");
    for (int j = 0; j < 4; ++j)
      if (overlap(rb[j], rs[j], bufs[i], bsz[i]))
        return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: the ring overlaps an input or the pool");
  }
  for (int j = 0; j < 4; ++j)
    if (overlap(rb[j], rs[j], o, o_b)) return fail(KDA_ERR_INVALID_ARG, "kda_fold_verify: the ring overlaps o");

  kda::VerifyArgs a{};
  a.batch = batch;
  a.n_tok = n_tok;
  a.n_heads = n_heads;
  a.n_layers = n_layers;
  a.layer = layer;
  a.n_slots = n_slots;
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.gk = in->gk;
  a.beta = in->beta;
  a.state_pool = state_pool;
  a.slot_idx = slot_idx;
  a.o = o;
  a.ring_k = ring->k;
  a.ring_v = ring->v;
  a.ring_gk = ring->gk;
  a.ring_beta = ring->beta;
  a.ring_len = ring->len;
  a.ring_start = ring_start;
  a.scale = scale;
  a.fold_len = fold_len;
  a.fold_start = fold_start;
  a.fold_pool = state_pool;
  const hipError_t e = kda::launch_fold_verify(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_fold_verify: launch", e);
  return ok();
}

kda_status kda_verify(int batch, int n_tok, int n_heads, int n_layers, int layer, int n_slots, kda_dtype qkv_dtype,
                      const kda_inputs* in, const float* state_pool, const int32_t* slot_idx, float* o,
                      const kda_ring* ring, const int32_t* ring_start, const int32_t* commit_len, float* commit_pool,
                      float scale, void* stream) {
  if (batch < 0 || n_tok < 1 || n_heads < 1 || n_layers < 1 || n_slots < 1 || layer < 0 || layer >= n_layers)
    return fail(KDA_ERR_INVALID_ARG, "kda_verify: bad batch/n_tok/n_heads/n_layers/layer/n_slots");
  if (qkv_dtype != KDA_BF16 && qkv_dtype != KDA_F32) return fail(KDA_ERR_INVALID_ARG, "kda_verify: bad qkv_dtype");
  if (qkv_dtype == KDA_F32 && ring)
    return fail(KDA_ERR_UNSUPPORTED, "kda_verify: the raw-input ring stores bf16 k/v; fp32 inputs need ring == NULL");
  if ((int64_t)batch * n_heads > 0x7fffffffLL) return fail(KDA_ERR_INVALID_ARG, "kda_verify: grid too large");
  if (batch == 0) return ok();
  if (!in || !in->q || !in->k || !in->v || !in->gk || !in->beta)
    return fail(KDA_ERR_INVALID_ARG, "kda_verify: q, k, v, gk and beta are required");
  if (!state_pool || !slot_idx || !o) return fail(KDA_ERR_INVALID_ARG, "kda_verify: state_pool, slot_idx and o are required");
  if ((commit_len == nullptr) != (commit_pool == nullptr))
    return fail(KDA_ERR_INVALID_ARG, "kda_verify: commit_len and commit_pool go together");
  if (ring) {
    if (!ring->k || !ring->v || !ring->gk || !ring->beta) return fail(KDA_ERR_INVALID_ARG, "kda_verify: ring buffers are NULL");
    if (!pow2(ring->len) || ring->len < 2 * n_tok)
      return fail(KDA_ERR_INVALID_ARG, "kda_verify: ring length must be a power of two >= 2 * n_tok");
  }
  const size_t esz = qkv_dtype == KDA_F32 ? 4 : 2;
  const size_t rows = (size_t)batch * n_tok * n_heads;
  const size_t pool_b = (size_t)n_slots * n_layers * n_heads * kState;
  const size_t o_b = rows * KDA_HEAD_DIM * 4;
  const size_t ring_units = (size_t)n_slots * n_layers * n_heads * (ring ? ring->len : 0);
  const void* bufs[] = {in->q, in->k, in->v, in->gk, in->beta, state_pool};
  const size_t bsz[] = {rows * KDA_HEAD_DIM * esz, rows * KDA_HEAD_DIM * esz, rows * KDA_HEAD_DIM * esz,
                        rows * KDA_HEAD_DIM * 4, rows * 4, pool_b};
  for (int i = 0; i < 6; ++i) {
    if (overlap(o, o_b, bufs[i], bsz[i])) return fail(KDA_ERR_INVALID_ARG, "kda_verify: o overlaps an input");
    if (commit_pool && commit_pool != state_pool && overlap(commit_pool, pool_b, bufs[i], bsz[i]))
      return fail(KDA_ERR_INVALID_ARG, "kda_verify: commit_pool overlaps an input or state_pool");
    if (ring) {
      const void* rb[] = {ring->k, ring->v, ring->gk, ring->beta};
      const size_t rs[] = {ring_units * KDA_HEAD_DIM * 2, ring_units * KDA_HEAD_DIM * 2, ring_units * KDA_HEAD_DIM * 4,
                           ring_units * 4};
      for (int j = 0; j < 4; ++j)
        if (overlap(rb[j], rs[j], bufs[i], bsz[i])) return fail(KDA_ERR_INVALID_ARG, "kda_verify: ring overlaps an input");
    }
  }
  if (commit_pool && overlap(commit_pool, pool_b, o, o_b))
    return fail(KDA_ERR_INVALID_ARG, "kda_verify: commit_pool overlaps o");

  kda::VerifyArgs a{};
  a.batch = batch;
  a.n_tok = n_tok;
  a.n_heads = n_heads;
  a.n_layers = n_layers;
  a.layer = layer;
  a.n_slots = n_slots;
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.gk = in->gk;
  a.beta = in->beta;
  a.state_pool = state_pool;
  a.slot_idx = slot_idx;
  a.o = o;
  if (ring) {
    a.ring_k = ring->k;
    a.ring_v = ring->v;
    a.ring_gk = ring->gk;
    a.ring_beta = ring->beta;
    a.ring_len = ring->len;
  }
  a.ring_start = ring_start;
  a.commit_len = commit_len;
  a.commit_pool = commit_pool;
  a.scale = scale;
  const hipError_t e = kda::launch_verify(a, qkv_dtype == KDA_F32, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_verify: launch", e);
  return ok();
}

kda_status kda_verify_ragged(int batch, int max_tok, int total_tok, int n_heads, int n_layers, int layer, int n_slots,
                             const kda_inputs* in, const int32_t* cu_tok, const float* state_pool,
                             const int32_t* slot_idx, float* o, const kda_ring* ring, const int32_t* ring_start,
                             float scale, void* stream) {
  if (batch < 0 || max_tok < 1 || max_tok > 16 || total_tok < 0 || n_heads < 1 || n_layers < 1 || n_slots < 1 ||
      layer < 0 || layer >= n_layers)
    return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: bad batch/max_tok/total_tok/n_heads/n_layers/layer/n_slots");
  if ((int64_t)batch * n_heads > 0x7fffffffLL || (int64_t)total_tok * n_heads * KDA_HEAD_DIM * 4 > 0x7fffffffLL)
    return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: too large");
  if (!cu_tok) return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: cu_tok is required");
  if (batch == 0 || total_tok == 0) return ok();
  if (!in || !in->q || !in->k || !in->v || !in->gk || !in->beta)
    return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: q, k, v, gk and beta are required");
  if (!state_pool || !slot_idx || !o)
    return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: state_pool, slot_idx and o are required");
  if (ring) {
    if (!ring->k || !ring->v || !ring->gk || !ring->beta)
      return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: ring buffers are NULL");
    if (!pow2(ring->len) || ring->len < 2 * max_tok)
      return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: ring length must be a power of two >= 2 * max_tok");
  }
  const size_t rows = (size_t)total_tok * n_heads;
  const size_t pool_b = (size_t)n_slots * n_layers * n_heads * kState;
  const size_t o_b = rows * KDA_HEAD_DIM * 4;
  const size_t ring_units = (size_t)n_slots * n_layers * n_heads * (ring ? ring->len : 0);
  const void* bufs[] = {in->q, in->k, in->v, in->gk, in->beta, state_pool, cu_tok};
  const size_t bsz[] = {rows * KDA_HEAD_DIM * 2, rows * KDA_HEAD_DIM * 2, rows * KDA_HEAD_DIM * 2,
                        rows * KDA_HEAD_DIM * 4, rows * 4, pool_b, ((size_t)batch + 1) * 4};
  for (int i = 0; i < 7; ++i) {
    if (overlap(o, o_b, bufs[i], bsz[i])) return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: o overlaps an input");
    if (ring) {
      const void* rb[] = {ring->k, ring->v, ring->gk, ring->beta};
      const size_t rs[] = {ring_units * KDA_HEAD_DIM * 2, ring_units * KDA_HEAD_DIM * 2, ring_units * KDA_HEAD_DIM * 4,
                           ring_units * 4};
      for (int j = 0; j < 4; ++j)
        if (overlap(rb[j], rs[j], bufs[i], bsz[i]))
          return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: ring overlaps an input");
    }
  }
  if (ring) {
    const void* rb[] = {ring->k, ring->v, ring->gk, ring->beta};
    const size_t rs[] = {ring_units * KDA_HEAD_DIM * 2, ring_units * KDA_HEAD_DIM * 2, ring_units * KDA_HEAD_DIM * 4,
                         ring_units * 4};
    for (int j = 0; j < 4; ++j)
      if (overlap(rb[j], rs[j], o, o_b)) return fail(KDA_ERR_INVALID_ARG, "kda_verify_ragged: the ring overlaps o");
  }
  kda::VerifyArgs a{};
  a.batch = batch;
  a.n_tok = max_tok;
  a.n_heads = n_heads;
  a.n_layers = n_layers;
  a.layer = layer;
  a.n_slots = n_slots;
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.gk = in->gk;
  a.beta = in->beta;
  a.state_pool = state_pool;
  a.slot_idx = slot_idx;
  a.o = o;
  if (ring) {
    a.ring_k = ring->k;
    a.ring_v = ring->v;
    a.ring_gk = ring->gk;
    a.ring_beta = ring->beta;
    a.ring_len = ring->len;
  }
  a.ring_start = ring_start;
  a.scale = scale;
  a.cu_tok = cu_tok;
  a.total_tok = total_tok;
  const hipError_t e = kda::launch_verify_chunk(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_verify_ragged: launch", e);
  return ok();
}

kda_status kda_prologue(int n_seq, int64_t total_tokens, int n_heads, int conv_width, const int32_t* cu_seqlens,
                        const void* xq, const void* xk, const void* xv, const float* conv_w, const void* conv_state_in,
                        void* conv_state_out, const float* b_raw, const float* g_raw, float eps, void* q, void* k,
                        void* v, float* beta, float* gk, void* stream) {
  if (n_seq < 0 || total_tokens < 0 || n_heads < 1 || conv_width < 1 || conv_width > 8)
    return fail(KDA_ERR_INVALID_ARG, "kda_prologue: bad n_seq/total_tokens/n_heads/conv_width");
  if (!(eps >= 0.f && eps < INFINITY)) return fail(KDA_ERR_INVALID_ARG, "kda_prologue: eps must be finite and >= 0");
  if (total_tokens > 0 && n_seq < 1) return fail(KDA_ERR_INVALID_ARG, "kda_prologue: tokens without sequences");
  if (n_heads > 0xffff) return fail(KDA_ERR_INVALID_ARG, "kda_prologue: n_heads must be <= 65535");
  if (total_tokens * n_heads > ((int64_t)1 << 33) || (int64_t)n_seq * 3 * (conv_width - 1) * n_heads * KDA_HEAD_DIM > ((int64_t)1 << 38))
    return fail(KDA_ERR_INVALID_ARG, "kda_prologue: too large");
  if (n_seq == 0) return ok();
  if (!cu_seqlens || !conv_w) return fail(KDA_ERR_INVALID_ARG, "kda_prologue: cu_seqlens and conv_w are required");
  if (total_tokens > 0 && (!xq || !xk || !xv || !b_raw || !g_raw || !q || !k || !v || !beta || !gk))
    return fail(KDA_ERR_INVALID_ARG, "kda_prologue: the projections, logits and outputs are required");
  {
    const void* al[11] = {xq, xk, xv, conv_w, conv_state_in, conv_state_out, g_raw, q, k, v, gk};
    for (const void* p : al)
      if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(KDA_ERR_INVALID_ARG, "kda_prologue: a row buffer is not 16-byte aligned");
  }
  const size_t rows = (size_t)total_tokens * n_heads;
  const size_t xb = rows * KDA_HEAD_DIM * 2, gb = rows * KDA_HEAD_DIM * 4, bb = rows * 4;
  const size_t stb = (size_t)n_seq * 3 * (conv_width - 1) * n_heads * KDA_HEAD_DIM * 2;
  const size_t wb = (size_t)3 * n_heads * KDA_HEAD_DIM * conv_width * 4;
  const void* ins[8] = {xq, xk, xv, conv_w, conv_state_in, b_raw, g_raw, cu_seqlens};
  const size_t insz[8] = {xb, xb, xb, wb, stb, bb, gb, ((size_t)n_seq + 1) * 4};
  const void* outs[6] = {q, k, v, beta, gk, conv_state_out};
  const size_t outsz[6] = {xb, xb, xb, bb, gb, stb};
  for (int o = 0; o < 6; ++o) {
    for (int i = 0; i < 8; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return fail(KDA_ERR_INVALID_ARG, "kda_prologue: an output overlaps an input");
    for (int o2 = o + 1; o2 < 6; ++o2)
      if (overlap(outs[o], outsz[o], outs[o2], outsz[o2])) return fail(KDA_ERR_INVALID_ARG, "kda_prologue: two outputs overlap");
  }
  kda::PrologueArgs a{};
  a.n_seq = n_seq;
  a.n_heads = n_heads;
  a.conv_width = conv_width;
  a.total_tokens = total_tokens;
  a.cu_seqlens = cu_seqlens;
  a.xq = static_cast<const uint16_t*>(xq);
  a.xk = static_cast<const uint16_t*>(xk);
  a.xv = static_cast<const uint16_t*>(xv);
  a.conv_w = conv_w;
  a.state_in = conv_width > 1 ? static_cast<const uint16_t*>(conv_state_in) : nullptr;
  a.state_out = conv_width > 1 ? static_cast<uint16_t*>(conv_state_out) : nullptr;
  a.b_raw = b_raw;
  a.g_raw = g_raw;
  a.eps = eps;
  a.q = static_cast<uint16_t*>(q);
  a.k = static_cast<uint16_t*>(k);
  a.v = static_cast<uint16_t*>(v);
  a.beta = beta;
  a.gk = gk;
  const hipError_t e = kda::launch_prologue(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_prologue: launch", e);
  return ok();
}

// ---------------------------------------------------------------------------------------------
// Measurement probes: the rates the chip reaches on the simplest work, for comparison with the
// kernels above in the same run. Grids of 256-thread workgroups: 32 per CU for the copy, 16 per CU
// for the read (or as many as its sink holds), two per CU for the MFMA loop (two waves per SIMD).

static int probe_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  return n;
}

kda_status kda_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst) return fail(KDA_ERR_INVALID_ARG, "kda_probe_copy: src and dst are required");
  if (bytes <= 0 || bytes % 16 != 0) return fail(KDA_ERR_INVALID_ARG, "kda_probe_copy: bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return fail(KDA_ERR_INVALID_ARG, "kda_probe_copy: src and dst must be 16-byte aligned");
  if (overlap(src, (size_t)bytes, dst, (size_t)bytes)) return fail(KDA_ERR_INVALID_ARG, "kda_probe_copy: src and dst overlap");
  const hipError_t e = kda::launch_probe_copy(src, dst, bytes / 16, 32 * probe_cus(), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_probe_copy: launch", e);
  return ok();
}

kda_status kda_probe_read(const void* src, int64_t bytes, float* sink, int64_t sink_floats, void* stream) {
  if (!src || !sink) return fail(KDA_ERR_INVALID_ARG, "kda_probe_read: src and sink are required");
  if (bytes <= 0 || bytes % 16 != 0) return fail(KDA_ERR_INVALID_ARG, "kda_probe_read: bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return fail(KDA_ERR_INVALID_ARG, "kda_probe_read: src must be 16-byte aligned");
  const int64_t grid = std::min<int64_t>(16LL * probe_cus(), sink_floats / 256);
  if (grid < 1) return fail(KDA_ERR_INVALID_ARG, "kda_probe_read: the sink must hold at least 256 floats");
  const hipError_t e = kda::launch_probe_read(src, bytes / 16, sink, (int)grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_probe_read: launch", e);
  return ok();
}

kda_status kda_probe_mfma(int iters, float seed, float* sink, int64_t sink_floats, int64_t* flop, void* stream) {
  if (iters < 1 || !sink || !flop) return fail(KDA_ERR_INVALID_ARG, "kda_probe_mfma: iters >= 1, sink and flop are required");
  const int64_t grid = std::min<int64_t>(2LL * probe_cus(), sink_floats / 256);
  if (grid < 1) return fail(KDA_ERR_INVALID_ARG, "kda_probe_mfma: the sink must hold at least 256 floats");
  // per workgroup: 4 waves x 8 accumulators x iters MFMAs of 2 x 16 x 16 x 32 flop (rounds run in
  // blocks of 32)
  if (iters > (1 << 30)) return fail(KDA_ERR_INVALID_ARG, "kda_probe_mfma: iters too large");
  iters = (iters + 31) / 32 * 32;
  *flop = grid * 4 * 8 * (int64_t)iters * (2 * 16 * 16 * 32);
  const hipError_t e = kda::launch_probe_mfma(iters, (int)grid, seed, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_probe_mfma: launch", e);
  return ok();
}

kda_status kda_state_move(int n_moves, const kda_move* moves, int n_slots, int64_t slot_floats, float* pool,
                          void* stream) {
  if (n_moves < 0 || n_slots < 1 || slot_floats < 4 || slot_floats % 4 != 0)
    return fail(KDA_ERR_INVALID_ARG, "kda_state_move: bad n_moves/n_slots/slot_floats (a positive multiple of 4)");
  if (n_moves == 0) return ok();
  if (!moves || !pool) return fail(KDA_ERR_INVALID_ARG, "kda_state_move: moves and pool are required");
  if (reinterpret_cast<uintptr_t>(pool) % 16 != 0) return fail(KDA_ERR_INVALID_ARG, "kda_state_move: pool is not 16-byte aligned");
  if ((uint64_t)slot_floats > (uint64_t)INT64_MAX / 4 / (uint64_t)n_slots) return fail(KDA_ERR_INVALID_ARG, "kda_state_move: pool too large");
  if (overlap(moves, (size_t)n_moves * sizeof(kda_move), pool, (size_t)n_slots * (size_t)slot_floats * 4))
    return fail(KDA_ERR_INVALID_ARG, "kda_state_move: moves overlaps the pool");
  const hipError_t e = kda::launch_state_move(n_moves, moves, n_slots, slot_floats, pool, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_state_move: launch", e);
  return ok();
}

kda_status kda_decode(int batch, int n_heads, int n_layers, int layer, int n_slots, int conv_width,
                      const void* xq, const void* xk, const void* xv, const float* conv_w, void* conv_state,
                      const float* b_raw, const float* g_raw, float* state_pool, const int32_t* slot_idx,
                      const void* gate, const float* norm_w, float qk_eps, float norm_eps, float scale, void* y,
                      float* o, void* stream) {
  if (batch < 0 || n_heads < 1 || n_heads > 0xffff || n_layers < 1 || layer < 0 || layer >= n_layers || n_slots < 1 ||
      conv_width < 1 || conv_width > 8)
    return fail(KDA_ERR_INVALID_ARG, "kda_decode: bad batch/n_heads/n_layers/layer/n_slots/conv_width");
  if (!(qk_eps >= 0.f && qk_eps < INFINITY) || !(norm_eps >= 0.f && norm_eps < INFINITY) || !std::isfinite(scale))
    return fail(KDA_ERR_INVALID_ARG, "kda_decode: eps values must be finite and >= 0, scale finite");
  if ((int64_t)batch * n_heads > 0x7fffffffLL) return fail(KDA_ERR_INVALID_ARG, "kda_decode: grid too large");
  if (batch == 0) return ok();
  if (!xq || !xk || !xv || !conv_w || !b_raw || !g_raw || !state_pool || !slot_idx || !gate || !norm_w || !y ||
      (conv_width > 1 && !conv_state))
    return fail(KDA_ERR_INVALID_ARG, "kda_decode: a required pointer is NULL");
  {
    const void* al[11] = {xq, xk, xv, conv_w, conv_state, g_raw, state_pool, gate, norm_w, y, o};
    for (const void* p : al)
      if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(KDA_ERR_INVALID_ARG, "kda_decode: a buffer is not 16-byte aligned");
  }
  const size_t rows = (size_t)batch * n_heads, HC = (size_t)n_heads * KDA_HEAD_DIM;
  const size_t xb = rows * KDA_HEAD_DIM * 2;
  const size_t csb = (size_t)batch * 3 * (conv_width - 1) * HC * 2;
  const size_t poolb = (size_t)n_slots * n_layers * n_heads * kState;
  const void* outs[4] = {conv_state, state_pool, y, o};
  const size_t outsz[4] = {csb, poolb, xb, rows * KDA_HEAD_DIM * 4};
  const void* ins[9] = {xq, xk, xv, conv_w, b_raw, g_raw, slot_idx, gate, norm_w};
  const size_t insz[9] = {xb, xb, xb, 3 * HC * conv_width * 4, rows * 4, rows * KDA_HEAD_DIM * 4, (size_t)batch * 4, xb,
                          (size_t)KDA_HEAD_DIM * 4};
  for (int a = 0; a < 4; ++a) {
    for (int i2 = 0; i2 < 9; ++i2)
      if (overlap(outs[a], outsz[a], ins[i2], insz[i2])) return fail(KDA_ERR_INVALID_ARG, "kda_decode: an output overlaps an input");
    for (int a2 = a + 1; a2 < 4; ++a2)
      if (overlap(outs[a], outsz[a], outs[a2], outsz[a2])) return fail(KDA_ERR_INVALID_ARG, "kda_decode: two outputs overlap");
  }
  kda::DecodeArgs d{};
  d.batch = batch;
  d.n_heads = n_heads;
  d.n_layers = n_layers;
  d.layer = layer;
  d.n_slots = n_slots;
  d.conv_width = conv_width;
  d.xq = static_cast<const uint16_t*>(xq);
  d.xk = static_cast<const uint16_t*>(xk);
  d.xv = static_cast<const uint16_t*>(xv);
  d.conv_w = conv_w;
  d.conv_state = static_cast<uint16_t*>(conv_state);
  d.b_raw = b_raw;
  d.g_raw = g_raw;
  d.state_pool = state_pool;
  d.slot_idx = slot_idx;
  d.gate = static_cast<const uint16_t*>(gate);
  d.norm_w = norm_w;
  d.qk_eps = qk_eps;
  d.norm_eps = norm_eps;
  d.scale = scale;
  d.y = static_cast<uint16_t*>(y);
  d.o = o;
  const hipError_t e = kda::launch_decode(d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_decode: launch", e);
  return ok();
}

kda_status kda_replay_fold(int batch, int n_heads, int n_layers, int n_slots, float* state_pool, const int32_t* slot_idx,
                           const kda_ring* ring, const int32_t* ring_start, const int32_t* accepted_len, void* stream) {
  if (batch < 0 || n_heads < 1 || n_layers < 1 || n_slots < 1)
    return fail(KDA_ERR_INVALID_ARG, "kda_replay_fold: bad batch/n_heads/n_layers/n_slots");
  if ((int64_t)batch * n_layers * n_heads > 0x7fffffffLL) return fail(KDA_ERR_INVALID_ARG, "kda_replay_fold: grid too large");
  if (batch == 0) return ok();
  if (!state_pool || !slot_idx || !accepted_len || !ring)
    return fail(KDA_ERR_INVALID_ARG, "kda_replay_fold: state_pool, slot_idx, ring and accepted_len are required");
  if (!ring->k || !ring->v || !ring->gk || !ring->beta) return fail(KDA_ERR_INVALID_ARG, "kda_replay_fold: ring buffers are NULL");
  if (!pow2(ring->len) || ring->len < 2) return fail(KDA_ERR_INVALID_ARG, "kda_replay_fold: ring length must be a power of two >= 2");
  const size_t pool_b = (size_t)n_slots * n_layers * n_heads * kState;
  const size_t ru = (size_t)n_slots * n_layers * n_heads * ring->len;
  const void* rb[] = {ring->k, ring->v, ring->gk, ring->beta};
  const size_t rs[] = {ru * KDA_HEAD_DIM * 2, ru * KDA_HEAD_DIM * 2, ru * KDA_HEAD_DIM * 4, ru * 4};
  for (int j = 0; j < 4; ++j)
    if (overlap(state_pool, pool_b, rb[j], rs[j])) return fail(KDA_ERR_INVALID_ARG, "kda_replay_fold: state_pool overlaps the ring");
  kda::FoldArgs a{};
  a.batch = batch;
  a.n_heads = n_heads;
  a.n_layers = n_layers;
  a.n_slots = n_slots;
  a.state_pool = state_pool;
  a.slot_idx = slot_idx;
  a.ring_k = ring->k;
  a.ring_v = ring->v;
  a.ring_gk = ring->gk;
  a.ring_beta = ring->beta;
  a.ring_len = ring->len;
  a.ring_start = ring_start;
  a.accepted_len = accepted_len;
  const hipError_t e = kda::launch_fold(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail("kda_replay_fold: launch", e);
  return ok();
}

}  // extern "C"
