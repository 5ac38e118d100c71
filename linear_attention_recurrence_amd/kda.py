"""Thin ctypes binding of libkda (include/kda.h): argument marshalling only.

Every function has the name of the C entry point it wraps and passes device
pointers of torch tensors plus the current HIP stream. Tensor shapes, dtypes
and contiguity are checked here against the layouts the header states, so a
kernel never addresses memory outside the tensors it was given. There is no
fallback: if libkda.so is missing or the HIP runtime is unavailable, calls
raise.

torch is imported before the library is loaded, so libkda binds to the HIP
runtime torch already mapped (both carry the soname libamdhip64.so.7) and
torch's stream handles are valid in it.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_DEVICE, KDA_ERR_HOST_ALLOC, KDA_ERR_NO_SLOT = 0, 1, 2, 3, 4, 5
KDA_SLOT_FREE, KDA_SLOT_TREE = -1, -2
KDA_BF16, KDA_F32 = 0, 1
KDA_PLAN_LPT, KDA_PLAN_FIFO = 0, 1
KDA_PREFILL_PLAN_RESIDENT = 1
KDA_HEAD_DIM = 128
KDA_CHUNK = 32

EXPORTS = ("kda_abi_version", "kda_last_error", "kda_plan_create", "kda_plan_create_ex", "kda_plan_v_blocks",
           "kda_plan_workspace_bytes", "kda_plan_num_items", "kda_plan_items", "kda_plan_upload", "kda_plan_destroy",
           "kda_host_release", "kda_chunk_prefill_noalloc",
           "kda_chunk_prefill", "kda_chunk_prefill_gated", "kda_gated_rmsnorm", "kda_prologue", "kda_verify",
           "kda_replay_fold", "kda_fold_verify", "kda_verify_ragged", "kda_state_move", "kda_chunk_split",
           "kda_slots_create", "kda_slots_destroy", "kda_slots_free_count", "kda_slots_owner", "kda_request_open",
           "kda_request_snapshot", "kda_request_donate", "kda_request_close", "kda_slot_release", "kda_decode",
           "kda_probe_copy", "kda_probe_read", "kda_probe_mfma")


class KdaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libkda status {status}: {msg}")
        self.status = status


class _Inputs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("gk", ctypes.c_void_p), ("beta", ctypes.c_void_p)]


class _Ring(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("gk", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("len", ctypes.c_int)]


class _Move(ctypes.Structure):
    _fields_ = [("src", ctypes.c_int32), ("dst", ctypes.c_int32)]


class RequestSlots(ctypes.Structure):
    """A request's slots (kda_request_slots): id, working slot, latest snapshot (-1 = none)."""
    _fields_ = [("id", ctypes.c_int32), ("working", ctypes.c_int32), ("snap", ctypes.c_int32)]


_lib = None


def lib():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.kda_abi_version.restype = i32
        L.kda_last_error.restype = ctypes.c_char_p
        L.kda_plan_create.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(vp)]
        L.kda_plan_create_ex.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(vp)]
        L.kda_plan_v_blocks.argtypes = [vp]
        L.kda_plan_v_blocks.restype = i32
        L.kda_plan_workspace_bytes.argtypes = [vp]
        L.kda_plan_workspace_bytes.restype = ctypes.c_size_t
        L.kda_plan_num_items.argtypes = [vp]
        L.kda_plan_num_items.restype = i32
        L.kda_plan_items.argtypes = [vp, vp]
        L.kda_plan_upload.argtypes = [vp, vp, vp]
        L.kda_plan_destroy.argtypes = [vp]
        L.kda_plan_destroy.restype = i32
        L.kda_host_release.argtypes = []
        L.kda_host_release.restype = i32
        L.kda_chunk_prefill.argtypes = [vp, ctypes.POINTER(_Inputs), vp, vp, vp, vp, i32, vp, vp, f32, i32, vp]
        L.kda_chunk_prefill_noalloc.argtypes = [vp, ctypes.POINTER(_Inputs), vp, vp, vp, vp, i32, vp, f32, vp]
        L.kda_chunk_prefill_gated.argtypes = [vp, ctypes.POINTER(_Inputs), vp, vp, f32, vp, vp, vp, vp, i32, vp, vp,
                                              f32, i32, vp]
        L.kda_gated_rmsnorm.argtypes = [ctypes.c_int64, vp, vp, vp, f32, vp, vp]
        L.kda_prologue.argtypes = [i32, ctypes.c_int64, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp,
                                   vp, vp, vp]
        L.kda_verify.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(_Inputs), vp, vp, vp,
                                 ctypes.POINTER(_Ring), vp, vp, vp, f32, vp]
        L.kda_replay_fold.argtypes = [i32, i32, i32, i32, vp, vp, ctypes.POINTER(_Ring), vp, vp, vp]
        L.kda_fold_verify.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(_Inputs), vp, vp, vp,
                                      ctypes.POINTER(_Ring), vp, vp, vp, f32, vp]
        L.kda_verify_ragged.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(_Inputs), vp, vp, vp, vp,
                                        ctypes.POINTER(_Ring), vp, f32, vp]
        i64 = ctypes.c_int64
        L.kda_state_move.argtypes = [i32, vp, i32, i64, vp, vp]
        L.kda_chunk_split.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64), i32, ctypes.POINTER(i32)]
        L.kda_slots_create.argtypes = [i32, ctypes.POINTER(vp)]
        L.kda_slots_destroy.argtypes = [vp]
        L.kda_slots_destroy.restype = None
        L.kda_slots_free_count.argtypes = [vp]
        L.kda_slots_free_count.restype = i32
        L.kda_slots_owner.argtypes = [vp, i32]
        L.kda_slots_owner.restype = i32
        L.kda_request_open.argtypes = [vp, i32, ctypes.POINTER(RequestSlots), ctypes.POINTER(_Move), ctypes.POINTER(i32)]
        L.kda_request_snapshot.argtypes = [vp, ctypes.POINTER(RequestSlots), ctypes.POINTER(_Move)]
        L.kda_request_donate.argtypes = [vp, ctypes.POINTER(RequestSlots), ctypes.POINTER(i32)]
        L.kda_request_close.argtypes = [vp, ctypes.POINTER(RequestSlots)]
        L.kda_slot_release.argtypes = [vp, i32]
        L.kda_decode.argtypes = [i32] * 6 + [vp] * 11 + [f32] * 3 + [vp] * 3
        L.kda_probe_copy.argtypes = [vp, vp, i64, vp]
        L.kda_probe_read.argtypes = [vp, i64, vp, i64, vp]
        L.kda_probe_mfma.argtypes = [i32, f32, vp, i64, ctypes.POINTER(i64), vp]
        for f in ("kda_probe_copy", "kda_probe_read", "kda_probe_mfma", "kda_decode", "kda_state_move", "kda_chunk_split", "kda_slots_create", "kda_request_open", "kda_request_snapshot",
                  "kda_request_donate", "kda_request_close", "kda_slot_release"):
            getattr(L, f).restype = i32
        for f in ("kda_plan_create", "kda_plan_create_ex", "kda_plan_items", "kda_plan_upload", "kda_chunk_prefill",
                  "kda_chunk_prefill_noalloc",
                  "kda_chunk_prefill_gated", "kda_gated_rmsnorm", "kda_prologue", "kda_verify", "kda_replay_fold",
                  "kda_fold_verify", "kda_verify_ragged"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _check(status):
    if status != KDA_OK:
        raise KdaError(status, lib().kda_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, shape, dtypes, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF, _F32, _I32 = (torch.bfloat16,), (torch.float32,), (torch.int32,)


def kda_abi_version():
    return lib().kda_abi_version()


def kda_last_error():
    return lib().kda_last_error().decode()


class Plan:
    """Owner of a kda_plan* (host data only). close() (or leaving a `with` block) destroys it; so does
    garbage collection. kda_plan_destroy makes no HIP call, so a finalizer that runs while a graph is
    being captured cannot disturb the capture (the pinned buffer is given back by a later
    kda_plan_create or kda_host_release)."""

    def __init__(self, handle, cu_seqlens, n_heads, snap_interval):
        self.handle = handle
        self.cu_seqlens = cu_seqlens
        self.n_seq = len(cu_seqlens) - 1
        self.n_heads = n_heads
        self.snap_interval = snap_interval
        self.total_tokens = int(cu_seqlens[-1])

    def close(self):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            _check(lib().kda_plan_destroy(h))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.kda_plan_destroy(h)  # status not raised from a finalizer


def kda_host_release():
    """Free the pinned buffers of destroyed plans (not during graph capture)."""
    _check(lib().kda_host_release())


def kda_plan_create(cu_seqlens_host, n_heads, snap_interval=0, order=KDA_PLAN_LPT, v_blocks=1):
    """kda_plan_create_ex: v_blocks = 1 or 2 value blocks per (sequence, head), 0 = by device size."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    h = ctypes.c_void_p()
    _check(lib().kda_plan_create_ex(cu.ctypes.data, len(cu) - 1, n_heads, snap_interval, order, v_blocks,
                                    ctypes.byref(h)))
    return Plan(h, cu.copy(), n_heads, snap_interval)


def kda_plan_v_blocks(plan):
    return int(lib().kda_plan_v_blocks(plan.handle))


def kda_plan_workspace_bytes(plan):
    return int(lib().kda_plan_workspace_bytes(plan.handle))


def kda_plan_num_items(plan):
    return int(lib().kda_plan_num_items(plan.handle))


def kda_plan_items(plan):
    out = np.zeros((kda_plan_num_items(plan), 4), dtype=np.int32)
    _check(lib().kda_plan_items(plan.handle, out.ctypes.data))
    return out


def kda_plan_upload(plan, workspace, stream=None):
    _need(workspace, "workspace", (kda_plan_workspace_bytes(plan),), (torch.uint8,))
    _check(lib().kda_plan_upload(plan.handle, _ptr(workspace), _stream(stream)))


def kda_chunk_prefill(plan, q, k, v, gk, beta, state_out, o, workspace, state_in=None, snap=None, snap_slots=0,
                      snap_count=None, scale=1.0, flags=0, stream=None):
    """Chunked prefill over the plan's THD-packed batch (see kda_chunk_prefill in include/kda.h)."""
    T, H, N, Dh = plan.total_tokens, plan.n_heads, plan.n_seq, KDA_HEAD_DIM
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (T, H, Dh), _BF)
    _need(gk, "gk", (T, H, Dh), _F32)
    _need(beta, "beta", (T, H), _F32)
    _need(o, "o", (T, H, Dh), _F32)
    _need(state_out, "state_out", (N, H, Dh, Dh), _F32)
    _need(state_in, "state_in", (N, H, Dh, Dh), _F32, allow_none=True)
    if snap is not None:
        _need(snap, "snap", (N, snap_slots, H, Dh, Dh), _F32)
    _need(snap_count, "snap_count", (N,), _I32, allow_none=True)
    _need(workspace, "workspace", (kda_plan_workspace_bytes(plan),), (torch.uint8,))
    ins = _Inputs(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(), beta.data_ptr())
    _check(lib().kda_chunk_prefill(plan.handle, ctypes.byref(ins), _ptr(state_in), _ptr(state_out), _ptr(o),
                                   _ptr(snap), int(snap_slots), _ptr(snap_count), _ptr(workspace), float(scale),
                                   int(flags), _stream(stream)))


KDA_NOALLOC_SCRATCH_BYTES = 1 << 20


def kda_chunk_prefill_noalloc(plan, q, k, v, gk, beta, state_out, o, state_in=None, snap=None, snap_slots=0,
                              snap_count=None, scale=1.0, stream=None):
    """kda_chunk_prefill without a workspace: the work list goes to the library's static device scratch
    (see kda_chunk_prefill_noalloc in include/kda.h). Allocates nothing."""
    T, H, N, Dh = plan.total_tokens, plan.n_heads, plan.n_seq, KDA_HEAD_DIM
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (T, H, Dh), _BF)
    _need(gk, "gk", (T, H, Dh), _F32)
    _need(beta, "beta", (T, H), _F32)
    _need(o, "o", (T, H, Dh), _F32)
    _need(state_out, "state_out", (N, H, Dh, Dh), _F32)
    _need(state_in, "state_in", (N, H, Dh, Dh), _F32, allow_none=True)
    if snap is not None:
        _need(snap, "snap", (N, snap_slots, H, Dh, Dh), _F32)
    _need(snap_count, "snap_count", (N,), _I32, allow_none=True)
    ins = _Inputs(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(), beta.data_ptr())
    _check(lib().kda_chunk_prefill_noalloc(plan.handle, ctypes.byref(ins), _ptr(state_in), _ptr(state_out), _ptr(o),
                                           _ptr(snap), int(snap_slots), _ptr(snap_count), float(scale),
                                           _stream(stream)))


def kda_chunk_prefill_gated(plan, q, k, v, gk, beta, gate, norm_w, eps, state_out, y, workspace, state_in=None,
                            snap=None, snap_slots=0, snap_count=None, scale=1.0, flags=0, stream=None):
    """Chunked prefill with the output gated RMSNorm fused in: writes bf16 y instead of fp32 o (see
    kda_chunk_prefill_gated in include/kda.h)."""
    T, H, N, Dh = plan.total_tokens, plan.n_heads, plan.n_seq, KDA_HEAD_DIM
    for name, t in (("q", q), ("k", k), ("v", v), ("gate", gate), ("y", y)):
        _need(t, name, (T, H, Dh), _BF)
    _need(gk, "gk", (T, H, Dh), _F32)
    _need(beta, "beta", (T, H), _F32)
    _need(norm_w, "norm_w", (Dh,), _F32)
    _need(state_out, "state_out", (N, H, Dh, Dh), _F32)
    _need(state_in, "state_in", (N, H, Dh, Dh), _F32, allow_none=True)
    if snap is not None:
        _need(snap, "snap", (N, snap_slots, H, Dh, Dh), _F32)
    _need(snap_count, "snap_count", (N,), _I32, allow_none=True)
    _need(workspace, "workspace", (kda_plan_workspace_bytes(plan),), (torch.uint8,))
    ins = _Inputs(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(), beta.data_ptr())
    _check(lib().kda_chunk_prefill_gated(plan.handle, ctypes.byref(ins), _ptr(gate), _ptr(norm_w), float(eps),
                                         _ptr(state_in), _ptr(state_out), _ptr(y), _ptr(snap), int(snap_slots),
                                         _ptr(snap_count), _ptr(workspace), float(scale), int(flags), _stream(stream)))


def kda_gated_rmsnorm(o, gate, norm_w, eps, y, stream=None):
    """The output gated RMSNorm over rows of 128 (see kda_gated_rmsnorm in include/kda.h); o fp32, gate and
    y bf16, all [..., 128] of the same shape, norm_w fp32 [128]."""
    Dh = KDA_HEAD_DIM
    if o.shape[-1] != Dh:
        raise ValueError(f"o has rows of {o.shape[-1]}, expected {Dh}")
    _need(o, "o", tuple(o.shape), _F32)
    _need(gate, "gate", tuple(o.shape), _BF)
    _need(y, "y", tuple(o.shape), _BF)
    _need(norm_w, "norm_w", (Dh,), _F32)
    _check(lib().kda_gated_rmsnorm(o.numel() // Dh, _ptr(o), _ptr(gate), _ptr(norm_w), float(eps), _ptr(y),
                                   _stream(stream)))


def kda_prologue(cu_seqlens, xq, xk, xv, conv_w, b_raw, g_raw, q, k, v, beta, gk, conv_state_in=None,
                 conv_state_out=None, eps=1e-6, stream=None):
    """The KDA prologue in one launch (see kda_prologue in include/kda.h): short conv + SiLU of the q/k/v
    projections with the conv-state carry, per-head L2 norm of q and k, beta = sigmoid, gk = -softplus.
    cu_seqlens is a device int32 tensor of n_seq + 1 prefix sums."""
    T, H, Dh = xq.shape[0], xq.shape[1], KDA_HEAD_DIM
    N = cu_seqlens.shape[0] - 1
    W = conv_w.shape[-1]
    for name, t in (("xq", xq), ("xk", xk), ("xv", xv), ("q", q), ("k", k), ("v", v)):
        _need(t, name, (T, H, Dh), _BF)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), _I32)
    _need(conv_w, "conv_w", (3, H * Dh, W), _F32)
    _need(b_raw, "b_raw", (T, H), _F32)
    _need(beta, "beta", (T, H), _F32)
    _need(g_raw, "g_raw", (T, H, Dh), _F32)
    _need(gk, "gk", (T, H, Dh), _F32)
    _need(conv_state_in, "conv_state_in", (N, 3, W - 1, H * Dh), _BF, allow_none=True)
    _need(conv_state_out, "conv_state_out", (N, 3, W - 1, H * Dh), _BF, allow_none=True)
    _check(lib().kda_prologue(N, T, H, W, _ptr(cu_seqlens), _ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_w),
                              _ptr(conv_state_in), _ptr(conv_state_out), _ptr(b_raw), _ptr(g_raw), float(eps), _ptr(q),
                              _ptr(k), _ptr(v), _ptr(beta), _ptr(gk), _stream(stream)))


def kda_decode(xq, xk, xv, conv_w, conv_state, b_raw, g_raw, state_pool, slot_idx, gate, norm_w, y, layer=0,
               o=None, qk_eps=1e-6, norm_eps=1e-6, scale=1.0, stream=None):
    """One decode step of a KDA layer in one launch (see kda_decode in include/kda.h): the prologue of each
    request's new token, the recurrent step with the commit in place, the output gated RMSNorm."""
    B, H, Dh = xq.shape[0], xq.shape[1], KDA_HEAD_DIM
    S, L = state_pool.shape[0], state_pool.shape[1]
    W = conv_w.shape[-1]
    for name, t in (("xq", xq), ("xk", xk), ("xv", xv), ("gate", gate), ("y", y)):
        _need(t, name, (B, H, Dh), _BF)
    _need(conv_w, "conv_w", (3, H * Dh, W), _F32)
    _need(conv_state, "conv_state", (B, 3, W - 1, H * Dh), _BF, allow_none=W == 1)
    _need(b_raw, "b_raw", (B, H), _F32)
    _need(g_raw, "g_raw", (B, H, Dh), _F32)
    _need(state_pool, "state_pool", (S, L, H, Dh, Dh), _F32)
    _need(slot_idx, "slot_idx", (B,), _I32)
    _need(norm_w, "norm_w", (Dh,), _F32)
    _need(o, "o", (B, H, Dh), _F32, allow_none=True)
    _check(lib().kda_decode(B, H, L, layer, S, W, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_w), _ptr(conv_state),
                            _ptr(b_raw), _ptr(g_raw), _ptr(state_pool), _ptr(slot_idx), _ptr(gate), _ptr(norm_w),
                            float(qk_eps), float(norm_eps), float(scale), _ptr(y), _ptr(o), _stream(stream)))


class Ring:
    """Device buffers of the per-slot raw-input ring: k, v bf16 [S, L, H, R, 128]; gk fp32; beta fp32 [S, L, H, R]."""

    def __init__(self, k, v, gk, beta):
        self.k, self.v, self.gk, self.beta = k, v, gk, beta
        self.len = k.shape[3]

    @staticmethod
    def empty(n_slots, n_layers, n_heads, length, device):
        sh = (n_slots, n_layers, n_heads, length, KDA_HEAD_DIM)
        return Ring(torch.empty(sh, dtype=torch.bfloat16, device=device),
                    torch.empty(sh, dtype=torch.bfloat16, device=device),
                    torch.empty(sh, dtype=torch.float32, device=device),
                    torch.empty(sh[:4], dtype=torch.float32, device=device))

    def check(self, n_slots, n_layers, n_heads):
        sh = (n_slots, n_layers, n_heads, self.len, KDA_HEAD_DIM)
        _need(self.k, "ring.k", sh, _BF)
        _need(self.v, "ring.v", sh, _BF)
        _need(self.gk, "ring.gk", sh, _F32)
        _need(self.beta, "ring.beta", sh[:4], _F32)

    def c(self):
        return _Ring(self.k.data_ptr(), self.v.data_ptr(), self.gk.data_ptr(), self.beta.data_ptr(), self.len)


def kda_verify(q, k, v, gk, beta, state_pool, slot_idx, o, layer, n_tok, ring=None, ring_start=None,
               commit_len=None, commit_pool=None, scale=1.0, stream=None):
    """Verify n_tok draft tokens of every request for one layer (see kda_verify in include/kda.h)."""
    S, L, H, Dh = state_pool.shape[0], state_pool.shape[1], state_pool.shape[2], KDA_HEAD_DIM
    B = slot_idx.shape[0]
    f32 = q.dtype == torch.float32
    qkv = _F32 if f32 else _BF
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (B * n_tok, H, Dh), qkv)
    _need(gk, "gk", (B * n_tok, H, Dh), _F32)
    _need(beta, "beta", (B * n_tok, H), _F32)
    _need(state_pool, "state_pool", (S, L, H, Dh, Dh), _F32)
    _need(slot_idx, "slot_idx", (B,), _I32)
    _need(o, "o", (B * n_tok, H, Dh), _F32)
    _need(ring_start, "ring_start", (B,), _I32, allow_none=True)
    _need(commit_len, "commit_len", (B,), _I32, allow_none=True)
    _need(commit_pool, "commit_pool", (S, L, H, Dh, Dh), _F32, allow_none=True)
    rc = None
    if ring is not None:
        ring.check(S, L, H)
        rc = ctypes.byref(ring.c())
    ins = _Inputs(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(), beta.data_ptr())
    _check(lib().kda_verify(B, n_tok, H, L, layer, S, KDA_F32 if f32 else KDA_BF16, ctypes.byref(ins),
                            _ptr(state_pool), _ptr(slot_idx), _ptr(o), rc, _ptr(ring_start), _ptr(commit_len),
                            _ptr(commit_pool), float(scale), _stream(stream)))


def kda_fold_verify(q, k, v, gk, beta, state_pool, slot_idx, o, layer, n_tok, ring, fold_len, fold_start=None,
                    ring_start=None, scale=1.0, stream=None):
    """Fold the previous window of `layer` into state_pool, then verify n_tok draft tokens from it
    (see kda_fold_verify in include/kda.h)."""
    S, L, H, Dh = state_pool.shape[0], state_pool.shape[1], state_pool.shape[2], KDA_HEAD_DIM
    B = slot_idx.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (B * n_tok, H, Dh), _BF)
    _need(gk, "gk", (B * n_tok, H, Dh), _F32)
    _need(beta, "beta", (B * n_tok, H), _F32)
    _need(state_pool, "state_pool", (S, L, H, Dh, Dh), _F32)
    _need(slot_idx, "slot_idx", (B,), _I32)
    _need(o, "o", (B * n_tok, H, Dh), _F32)
    _need(fold_len, "fold_len", (B,), _I32)
    _need(fold_start, "fold_start", (B,), _I32, allow_none=True)
    _need(ring_start, "ring_start", (B,), _I32, allow_none=True)
    ring.check(S, L, H)
    ins = _Inputs(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(), beta.data_ptr())
    _check(lib().kda_fold_verify(B, n_tok, H, L, layer, S, ctypes.byref(ins), _ptr(state_pool), _ptr(slot_idx),
                                 _ptr(o), ctypes.byref(ring.c()), _ptr(fold_start), _ptr(fold_len), _ptr(ring_start),
                                 float(scale), _stream(stream)))


def kda_verify_ragged(q, k, v, gk, beta, cu_tok, state_pool, slot_idx, o, layer, max_tok, ring=None, ring_start=None,
                      scale=1.0, stream=None):
    """Verify each request's own trimmed window of draft tokens for one layer; the windows are packed
    back to back, request b's at rows cu_tok[b] .. cu_tok[b + 1] - 1 (see kda_verify_ragged in
    include/kda.h). cu_tok is a device int32 tensor of batch + 1 prefix sums."""
    S, L, H, Dh = state_pool.shape[0], state_pool.shape[1], state_pool.shape[2], KDA_HEAD_DIM
    B = slot_idx.shape[0]
    total = q.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (total, H, Dh), _BF)
    _need(gk, "gk", (total, H, Dh), _F32)
    _need(beta, "beta", (total, H), _F32)
    _need(cu_tok, "cu_tok", (B + 1,), _I32)
    _need(state_pool, "state_pool", (S, L, H, Dh, Dh), _F32)
    _need(slot_idx, "slot_idx", (B,), _I32)
    _need(o, "o", (total, H, Dh), _F32)
    _need(ring_start, "ring_start", (B,), _I32, allow_none=True)
    rc = None
    if ring is not None:
        ring.check(S, L, H)
        rc = ctypes.byref(ring.c())
    ins = _Inputs(q.data_ptr(), k.data_ptr(), v.data_ptr(), gk.data_ptr(), beta.data_ptr())
    _check(lib().kda_verify_ragged(B, max_tok, total, H, L, layer, S, ctypes.byref(ins), _ptr(cu_tok), _ptr(state_pool),
                                   _ptr(slot_idx), _ptr(o), rc, _ptr(ring_start), float(scale), _stream(stream)))


def kda_replay_fold(state_pool, slot_idx, ring, accepted_len, ring_start=None, stream=None):
    """Fold the accepted prefix of every request into state_pool, in place (see include/kda.h)."""
    S, L, H, Dh = state_pool.shape[0], state_pool.shape[1], state_pool.shape[2], KDA_HEAD_DIM
    B = slot_idx.shape[0]
    _need(state_pool, "state_pool", (S, L, H, Dh, Dh), _F32)
    _need(slot_idx, "slot_idx", (B,), _I32)
    _need(accepted_len, "accepted_len", (B,), _I32)
    _need(ring_start, "ring_start", (B,), _I32, allow_none=True)
    ring.check(S, L, H)
    _check(lib().kda_replay_fold(B, H, L, S, _ptr(state_pool), _ptr(slot_idx), ctypes.byref(ring.c()),
                                 _ptr(ring_start), _ptr(accepted_len), _stream(stream)))


# ---------------------------------------------------------------- prefix-cache state moves
def kda_state_move(pool, moves, stream=None):
    """Whole-slot copies pool[src] -> pool[dst] for each row (src, dst) of moves, in one launch (see
    include/kda.h). pool: fp32 [n_slots, ...] contiguous; moves: int32 [n, 2] on the device (an empty
    tensor: nothing to do)."""
    if moves.numel() == 0:
        return
    if moves.dim() != 2 or moves.shape[1] != 2:
        raise ValueError("moves must be int32 [n, 2]")
    _need(moves, "moves", tuple(moves.shape), _I32)
    if pool.dim() < 2:
        raise ValueError("pool must be [n_slots, ...]")
    _need(pool, "pool", tuple(pool.shape), _F32)
    _check(lib().kda_state_move(moves.shape[0], _ptr(moves), pool.shape[0], pool[0].numel(), _ptr(pool),
                                _stream(stream)))


# ---------------------------------------------------------------- measurement probes
def kda_probe_copy(dst, src, stream=None):
    """dst = src through the library's streaming copy probe (see include/kda.h). Both contiguous device
    tensors of the same number of bytes (a multiple of 16)."""
    nb = src.numel() * src.element_size()
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()) or dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst must be contiguous device tensors of the same size in bytes")
    _check(lib().kda_probe_copy(_ptr(src), _ptr(dst), nb, _stream(stream)))


def kda_probe_read(src, sink, stream=None):
    """Reads src once through the streaming read probe; sink: fp32 device tensor of >= 256 elements
    receiving one partial sum per thread (their total is the sum of src's fp32 values)."""
    if not (src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous device tensor")
    _need(sink, "sink", tuple(sink.shape), _F32)
    _check(lib().kda_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), sink.numel(), _stream(stream)))


def kda_probe_mfma(iters, sink, seed=1e-3, stream=None):
    """Runs the bf16 MFMA loop probe; sink: fp32 device tensor of >= 256 elements. Returns the flops of
    the launch."""
    _need(sink, "sink", tuple(sink.shape), _F32)
    flop = ctypes.c_int64(0)
    _check(lib().kda_probe_mfma(int(iters), float(seed), _ptr(sink), sink.numel(), ctypes.byref(flop), _stream(stream)))
    return int(flop.value)


def kda_chunk_split(pos0, length, budget, align=256):
    """Checkpoint-aligned chunk lengths for an extend of `length` tokens after `pos0` (see include/kda.h)."""
    n = ctypes.c_int32(0)
    st = lib().kda_chunk_split(pos0, length, budget, align, None, 0, ctypes.byref(n))  # counts the chunks
    if st != KDA_OK and n.value == 0:
        _check(st)
    buf = (ctypes.c_int64 * max(n.value, 1))()
    _check(lib().kda_chunk_split(pos0, length, budget, align, buf, n.value, ctypes.byref(n)))
    return [int(buf[i]) for i in range(n.value)]


class SlotPool:
    """Ownership of a state pool's slots under the three state moves (kda_slots in include/kda.h). Host
    only: the moves it returns are enqueued with kda_state_move on the forward stream."""

    def __init__(self, n_slots):
        h = ctypes.c_void_p()
        _check(lib().kda_slots_create(n_slots, ctypes.byref(h)))
        self._h = h
        self.n_slots = n_slots

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.kda_slots_destroy(self._h)
            self._h = None

    def free_count(self):
        return lib().kda_slots_free_count(self._h)

    def owner(self, slot):
        return lib().kda_slots_owner(self._h, slot)

    def open(self, cached_slot=-1):
        """-> (RequestSlots, [(src, dst)]): the working slot, and the copy-on-write move if restoring."""
        r, mv, n = RequestSlots(), _Move(), ctypes.c_int32(0)
        _check(lib().kda_request_open(self._h, cached_slot, ctypes.byref(r), ctypes.byref(mv), ctypes.byref(n)))
        return r, ([(mv.src, mv.dst)] if n.value else [])

    def snapshot(self, r):
        mv = _Move()
        _check(lib().kda_request_snapshot(self._h, ctypes.byref(r), ctypes.byref(mv)))
        return (mv.src, mv.dst)

    def donate(self, r):
        slot = ctypes.c_int32(-1)
        _check(lib().kda_request_donate(self._h, ctypes.byref(r), ctypes.byref(slot)))
        return slot.value

    def close(self, r):
        _check(lib().kda_request_close(self._h, ctypes.byref(r)))

    def release(self, slot):
        _check(lib().kda_slot_release(self._h, slot))
