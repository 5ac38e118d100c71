"""Device build of the generator: fills torch device tensors with the same values
the host build (synth.rows) produces, bit for bit.

torch is imported first so libsynth_gpu.so binds to the HIP runtime torch mapped.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import BF16, F32, F64, NEG_SOFTPLUS, NORMAL, SIGMOID, UNIT_ROW, D
from . import T_Q, T_K, T_V, T_GK, T_BETA, T_STATE  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth_gpu.so")
_lib = None
_DT = {torch.float64: F64, torch.float32: F32, torch.bfloat16: BF16}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(_LIB_PATH)
        L.synth_gpu_fill.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                     ctypes.c_void_p, ctypes.c_void_p]
        L.synth_gpu_fill.restype = ctypes.c_int
        _lib = L
    return _lib


def fill(t, seed, tid, sub, kind, row_start=0, row_step=1, row_len=D, scale=1.0):
    """Fill contiguous device tensor t ([n_rows * row_len] elements) with rows
    row_start + i*row_step of the logical tensor (seed, tid, sub)."""
    assert t.is_cuda and t.is_contiguous() and t.dtype in _DT
    assert t.numel() % row_len == 0
    n_rows = t.numel() // row_len
    rc = lib().synth_gpu_fill(seed, tid, sub, kind, _DT[t.dtype], row_start, row_step, n_rows, row_len,
                              float(scale), ctypes.c_void_p(t.data_ptr()),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill failed ({rc})")
    return t


def prefill_inputs(seed, T, H, device, qkv_dtype=torch.bfloat16, tids=(T_Q, T_K, T_V, T_GK, T_BETA), sub=0):
    """q, k, v [T, H, 128] (qkv_dtype), gk [T, H, 128] fp32, beta [T, H] fp32 on device."""
    tq, tk, tv, tg, tb = tids
    q = fill(torch.empty((T, H, D), dtype=qkv_dtype, device=device), seed, tq, sub, UNIT_ROW)
    k = fill(torch.empty((T, H, D), dtype=qkv_dtype, device=device), seed, tk, sub, UNIT_ROW)
    v = fill(torch.empty((T, H, D), dtype=qkv_dtype, device=device), seed, tv, sub, NORMAL)
    gk = fill(torch.empty((T, H, D), dtype=torch.float32, device=device), seed, tg, sub, NEG_SOFTPLUS)
    beta = fill(torch.empty((T, H), dtype=torch.float32, device=device), seed, tb, sub, SIGMOID, row_len=1)
    return q, k, v, gk, beta


def gate(seed, T, H, device, sub=0):
    """Output-gate values [T, H, 128] bf16 on device (the rows synth.gate_rows gives on the host)."""
    from . import T_GATE
    return fill(torch.empty((T, H, D), dtype=torch.bfloat16, device=device), seed, T_GATE, sub, NORMAL)


def states(seed, n_units, device, tid=T_STATE, sub=0, sigma=0.1, out=None):
    """n_units states N(0, sigma^2) as [n_units, 128, 128] fp32 (unit u = rows u*128 ..)."""
    if out is None:
        out = torch.empty((n_units, D, D), dtype=torch.float32, device=device)
    return fill(out, seed, tid, sub, NORMAL, scale=sigma)
