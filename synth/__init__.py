"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds input distributions only -- none of the recurrence's
arithmetic. Every element is a pure function of (seed, tensor id, sub-tensor
id, flat index), drawn with Philox-4x32-10 (Salmon et al., SC'11) and the
Box-Muller transform, computed in fp64 and rounded to the storage type
(fp32 by round-to-nearest-even, bf16 by round-to-nearest-even directly from
fp64). The C source is ``synth/synth.c``; build it with
``__graft_entry__.build()``.

Workload recipes (shapes follow the pages: K = V = 128, H64/H96 heads, extend
lengths 64..24576, 69 KDA layers, gamma + 1 = 8 draft tokens, accept length
about 2.7, a 1M-token context):

* q, k ~ N(0, 1) per element, then L2-normalised per (token, head) row in fp64;
* v ~ N(0, 1);
* gk = -softplus(z), z ~ N(0, 1)  (per-token, per-key-channel log-decay <= 0);
* beta = sigmoid(z), z ~ N(0, 1);
* initial / committed states ~ N(0, 0.1^2) where a workload has one.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

NORMAL, UNIT_ROW, NEG_SOFTPLUS, SIGMOID = 0, 1, 2, 3
F64, F32, BF16 = 0, 1, 2
_NP = {F64: np.float64, F32: np.float32, BF16: np.uint16}

# tensor ids
T_Q, T_K, T_V, T_GK, T_BETA, T_STATE, T_LENS, T_ACCEPT = 1, 2, 3, 4, 5, 6, 7, 8
T_WINDOW = 9
T_GATE, T_NORMW = 10, 16  # inputs of the output gated RMSNorm
T_DEC_Q, T_DEC_K, T_DEC_V, T_DEC_GK, T_DEC_BETA = 11, 12, 13, 14, 15

D = 128  # K = V = 128


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(_LIB_PATH)
        L.synth_fill.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int, ctypes.c_double, ctypes.c_void_p]
        L.synth_fill.restype = ctypes.c_int
        L.synth_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_void_p]
        L.synth_uniform.restype = ctypes.c_int
        L.synth_round_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.synth_round_bf16.restype = None
        L.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.synth_philox4x32_10.restype = None
        L.synth_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def rows(seed, tid, sub, kind, dtype, row_start, row_step, n_rows, row_len=D, scale=1.0, out=None):
    """Rows r = row_start + i*row_step (i < n_rows) of the logical tensor, as [n_rows, row_len]."""
    if out is None:
        out = np.empty((n_rows, row_len), dtype=_NP[dtype])
    assert out.flags.c_contiguous and out.size == n_rows * row_len and out.dtype == _NP[dtype]
    rc = lib().synth_fill(seed, tid, sub, kind, dtype, row_start, row_step, n_rows, row_len,
                          float(scale), out.ctypes.data)
    if rc != 0:
        raise ValueError("synth_fill rejected its arguments")
    return out


def tensor(seed, tid, sub, kind, dtype, shape, row_len=D, scale=1.0, out=None):
    """A whole tensor of `shape` whose last dimension is the row (row_len)."""
    n = int(np.prod(shape))
    assert n % row_len == 0
    arr = rows(seed, tid, sub, kind, dtype, 0, 1, n // row_len, row_len, scale,
               out=None if out is None else out.reshape(-1, row_len))
    return arr.reshape(shape)


def uniform(seed, tid, sub, n, start=0):
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform(seed, tid, sub, start, n, out.ctypes.data)
    return out


def round_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().synth_round_bf16(x.ctypes.data, y.ctypes.data, x.size)
    return y


def bf16_to_f64(h):
    """Exact widening of bf16 bit patterns (uint16) to fp64."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- workload recipes ------------------------------------------------------

def loguniform_lengths(seed, n, lo=64, hi=24576):
    """Extend lengths L = clamp(round(exp(U(ln lo, ln hi))), lo, hi)."""
    u = uniform(seed, T_LENS, 0, n)
    x = np.exp(math.log(lo) + (1.0 - u) * (math.log(hi) - math.log(lo)))
    return np.clip(np.floor(x + 0.5), lo, hi).astype(np.int64)


def geometric_accept(seed, n, mean=2.7, cap=8):
    """Accepted lengths: geometric on {1, 2, ...} with p = 1/mean, clipped to cap."""
    p = 1.0 / mean
    u = uniform(seed, T_ACCEPT, 0, n)
    g = 1 + np.floor(np.log(u) / math.log(1.0 - p))
    return np.minimum(cap, g).astype(np.int64)


def trimmed_windows(seed, n, cap=8):
    """Verify windows kept by a per-request trimming planner: uniform on {1, ..., cap}. The pages give
    no distribution for the trimmed lengths; this spreads the windows over the whole range."""
    u = uniform(seed, T_WINDOW, 0, n)
    return np.minimum(cap, 1 + np.floor(u * cap)).astype(np.int64)


PREFILL_CONFIGS = {
    # name: (seed, lengths spec, heads, qkv dtype, initial state, snap interval, snap slots)
    "single_64": dict(seed=0, N=1, lengths=[64], H=1, state_in="zero", snap_interval=0, snap_slots=0),
    "prefill_4x2048_h64": dict(seed=1, N=4, lengths=[2048] * 4, H=64, state_in="normal", snap_interval=0, snap_slots=0),
    "varlen_h96": dict(seed=2, N=32, lengths="loguniform", H=96, state_in=None, snap_interval=2048, snap_slots=2),
    "long_1m_h96": dict(seed=4, N=1, lengths=[1048576], H=96, state_in=None, snap_interval=4096, snap_slots=2),
}

VERIFY_CONFIG = dict(seed=3, B=256, L=69, H=8, T=8, R=16, accept_mean=2.7)
DECODE_STEPS = 128  # single-token decode steps after the long prefill


def prefill_lengths(cfg):
    c = PREFILL_CONFIGS[cfg] if isinstance(cfg, str) else cfg
    if isinstance(c["lengths"], str):
        return loguniform_lengths(c["seed"], c["N"])
    return np.asarray(c["lengths"], dtype=np.int64)


def cu_seqlens(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    assert cu[-1] < 2 ** 31
    return cu.astype(np.int32)


def prefill_rows(seed, H, t0, nt, h=None, qkv_dtype=BF16, tids=(T_Q, T_K, T_V, T_GK, T_BETA), sub=0):
    """Inputs for tokens [t0, t0+nt) of a packed [T, H, 128] batch.

    With h=None: all heads, arrays [nt, H, 128] (beta [nt, H]).
    With h given: that head only, arrays [nt, 128] (beta [nt]).
    """
    tq, tk, tv, tg, tb = tids
    if h is None:
        r0, step, n = t0 * H, 1, nt * H
        shp, bshp = (nt, H, D), (nt, H)
    else:
        r0, step, n = t0 * H + h, H, nt
        shp, bshp = (nt, D), (nt,)
    q = rows(seed, tq, sub, UNIT_ROW, qkv_dtype, r0, step, n).reshape(shp)
    k = rows(seed, tk, sub, UNIT_ROW, qkv_dtype, r0, step, n).reshape(shp)
    v = rows(seed, tv, sub, NORMAL, qkv_dtype, r0, step, n).reshape(shp)
    gk = rows(seed, tg, sub, NEG_SOFTPLUS, F32, r0, step, n).reshape(shp)
    beta = rows(seed, tb, sub, SIGMOID, F32, r0, step, n, row_len=1).reshape(bshp)
    return q, k, v, gk, beta


def gate_rows(seed, H, t0, nt, h=None, sub=0):
    """Output-gate values N(0,1) in bf16 for tokens [t0, t0+nt) of a packed [T, H, 128] batch (indexed like
    prefill_rows; with h given, that head only). The pages give no distribution for the gate."""
    if h is None:
        r0, step, n, shp = t0 * H, 1, nt * H, (nt, H, D)
    else:
        r0, step, n, shp = t0 * H + h, H, nt, (nt, D)
    return rows(seed, T_GATE, sub, NORMAL, BF16, r0, step, n).reshape(shp)


def norm_weight(seed):
    """Per-channel weights of the output norm, fp32(1 + 0.1 N(0,1)) (the pages give none)."""
    x = rows(seed, T_NORMW, 0, NORMAL, F64, 0, 1, 1)
    return (1.0 + 0.1 * x.reshape(D)).astype(np.float32)


def state_rows(seed, unit0, n_units, unit_step=1, tid=T_STATE, sub=0, sigma=0.1, dtype=F32):
    """States N(0, sigma^2) for units unit0 + i*unit_step, as [n_units, 128, 128]."""
    out = np.empty((n_units, D, D), dtype=_NP[dtype])
    if unit_step == 1:
        rows(seed, tid, sub, NORMAL, dtype, unit0 * D, 1, n_units * D, D, sigma, out=out.reshape(-1, D))
    else:
        for i in range(n_units):
            rows(seed, tid, sub, NORMAL, dtype, (unit0 + i * unit_step) * D, 1, D, D, sigma, out=out[i])
    return out
