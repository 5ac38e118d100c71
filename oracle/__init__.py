"""fp64 CPU oracle for the KDA gated delta-rule recurrence -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package. The product path (the HIP library and its Python
binding) never touches it, and the two share no code.

The arithmetic lives in ``oracle/oracle.c`` (built into ``liboracle.so`` by
``__graft_entry__.build()``); this module only marshals numpy arrays. Inputs
of any stored dtype are widened exactly to fp64 (bf16 bit patterns given as
uint16, fp32, fp64).

Parity pins: every function here is checked in ``tests/test_oracle.py``
against closed forms, invariants, a brute-force matrix form on tiny shapes
and an independently derived chunked algebra. The pages print no worked
example and no output value, so absolute outputs are parity unpinned by the
pages themselves; for the output gated RMSNorm and the prologue even the
formulas are readings (the pages name the operations only), pinned by those
invariants alone.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.kda_oracle_recurrent.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, dbl, vp, vp, i64, i64,
                                           i32, vp, vp]
        L.kda_oracle_verify.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, dbl, vp, vp, i32, vp, vp,
                                        vp, vp, vp]
        L.kda_oracle_fold.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.kda_oracle_chunked.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp, dbl, vp, vp]
        L.kda_oracle_gated_rmsnorm.argtypes = [i64, i32, vp, vp, vp, dbl, vp]
        L.kda_oracle_prologue.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, dbl, vp, vp, vp, vp, vp, vp]
        for f in (L.kda_oracle_recurrent, L.kda_oracle_verify, L.kda_oracle_fold, L.kda_oracle_chunked,
                  L.kda_oracle_gated_rmsnorm, L.kda_oracle_prologue):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def f64(x):
    """Exact widening to a C-contiguous fp64 array (uint16 = bf16 bit patterns)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data


def recurrent(q, k, v, gk, beta, S0=None, scale=1.0, want_o=True, pos0=0, snap_interval=0,
              snap_slots=0, snaps=None):
    """Token-by-token recurrence for one unit.

    q, k, gk: [L, K]; v: [L, V]; beta: [L]; S0: [K, V] or None (zeros).
    Returns (o [L, V] or None, S_end [K, V], snaps [slots, K, V] or None, n_snapshots).
    """
    q, k, v, gk, beta = (f64(a) for a in (q, k, v, gk, beta))
    L, K = k.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if S0 is None else f64(S0).copy()
    o = np.empty((L, V)) if want_o else None
    if snap_interval > 0:
        if snaps is None:
            snaps = np.zeros((snap_slots, K, V))
        assert snaps.dtype == np.float64 and snaps.flags.c_contiguous
    cnt = np.zeros(1, dtype=np.int64)
    rc = lib().kda_oracle_recurrent(L, K, V, _p(q), _p(k), _p(v), _p(gk), _p(beta), float(scale),
                                    _p(S), _p(o), pos0, snap_interval, snap_slots,
                                    _p(snaps) if snap_interval > 0 else None, cnt.ctypes.data)
    if rc != 0:
        raise ValueError("kda_oracle_recurrent rejected its arguments")
    return o, S, (snaps if snap_interval > 0 else None), int(cnt[0])


def verify(q, k, v, gk, beta, S0, scale=1.0, commit_len=0, record=True):
    """Verify n_tok steps from a copy of S0 (never written).

    Returns (o [n, V], S_commit [K, V] or None, ring dict of recorded (k, v, gk, beta) or None).
    """
    q, k, v, gk, beta = (f64(a) for a in (q, k, v, gk, beta))
    n, K = k.shape
    V = v.shape[1]
    S0 = f64(S0)
    o = np.empty((n, V))
    Sc = np.empty((K, V)) if commit_len > 0 else None
    ring = None
    if record:
        ring = dict(k=np.empty((n, K)), v=np.empty((n, V)), gk=np.empty((n, K)), beta=np.empty(n))
    r = ring or {}
    rc = lib().kda_oracle_verify(n, K, V, _p(q), _p(k), _p(v), _p(gk), _p(beta), float(scale), _p(S0),
                                 _p(o), commit_len, _p(Sc), _p(r.get("k")), _p(r.get("v")),
                                 _p(r.get("gk")), _p(r.get("beta")))
    if rc != 0:
        raise ValueError("kda_oracle_verify rejected its arguments")
    return o, Sc, ring


def fold(n, ring_k, ring_v, ring_gk, ring_beta, S):
    """Advance S ([K, V] fp64, modified in place and returned) by the first n recorded steps."""
    ring_k, ring_v, ring_gk, ring_beta = (f64(a) for a in (ring_k, ring_v, ring_gk, ring_beta))
    assert S.dtype == np.float64 and S.flags.c_contiguous
    K, V = S.shape
    rc = lib().kda_oracle_fold(int(n), K, V, _p(ring_k), _p(ring_v), _p(ring_gk), _p(ring_beta), _p(S))
    if rc != 0:
        raise ValueError("kda_oracle_fold rejected its arguments")
    return S


def chunked(q, k, v, gk, beta, S0=None, scale=1.0, chunk=64):
    """The chunked (WY) form of the same recurrence; returns (o, S_end)."""
    q, k, v, gk, beta = (f64(a) for a in (q, k, v, gk, beta))
    L, K = k.shape
    V = v.shape[1]
    S = np.zeros((K, V)) if S0 is None else f64(S0).copy()
    o = np.empty((L, V))
    rc = lib().kda_oracle_chunked(L, K, V, chunk, _p(q), _p(k), _p(v), _p(gk), _p(beta), float(scale),
                                  _p(S), _p(o))
    if rc != 0:
        raise ValueError("kda_oracle_chunked rejected its arguments")
    return o, S


def gated_rmsnorm(o, g, w, eps):
    """Output gated RMSNorm over the last axis (rows of V): o / sqrt(mean(o^2) + eps) * w * sigmoid(g)."""
    o, g, w = f64(o), f64(g), f64(w)
    V = o.shape[-1]
    if g.shape != o.shape or w.shape != (V,):
        raise ValueError("gated_rmsnorm: g must match o, w must have the row length")
    y = np.empty_like(o)
    rc = lib().kda_oracle_gated_rmsnorm(o.size // V, V, _p(o), _p(g), _p(w), float(eps), _p(y))
    if rc != 0:
        raise ValueError("kda_oracle_gated_rmsnorm rejected its arguments")
    return y


def prologue(xq, xk, xv, conv_w, state_in, b_raw, g_raw, eps):
    """The KDA prologue of one sequence: xq, xk, xv [L, H, 128]; conv_w [3, H*128, W]; state_in
    [3, W-1, H*128]; b_raw [L, H]; g_raw [L, H, 128]. Returns q, k, v [L, H, 128], beta [L, H],
    gk [L, H, 128] and state_out [3, W-1, H*128], all fp64."""
    xq, xk, xv, conv_w, state_in, b_raw, g_raw = (f64(a) for a in (xq, xk, xv, conv_w, state_in, b_raw, g_raw))
    L, H = xq.shape[0], xq.shape[1]
    W = conv_w.shape[2]
    if conv_w.shape != (3, H * 128, W) or state_in.shape != (3, W - 1, H * 128):
        raise ValueError("prologue: conv_w must be [3, H*128, W] and state_in [3, W-1, H*128]")
    q, k, v = (np.empty((L, H, 128)) for _ in range(3))
    beta, gk = np.empty((L, H)), np.empty((L, H, 128))
    state_out = np.empty((3, W - 1, H * 128))
    rc = lib().kda_oracle_prologue(L, H, W, _p(xq), _p(xk), _p(xv), _p(conv_w), _p(state_in), _p(b_raw), _p(g_raw),
                                   float(eps), _p(q), _p(k), _p(v), _p(beta), _p(gk), _p(state_out))
    if rc != 0:
        raise ValueError("kda_oracle_prologue rejected its arguments")
    return q, k, v, beta, gk, state_out


def run_parallel(fn, items, threads=None):
    """Map fn over independent units on a thread pool (the C calls release the GIL)."""
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))
