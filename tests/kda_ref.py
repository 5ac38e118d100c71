"""Helpers for the GPU parity tests: oracle runs on host-regenerated inputs and
the error measure.

Inputs on both sides come from the seeded generator (synth/): the device build
fills the GPU tensors, the host build regenerates exactly the slices the
oracle needs (the two builds agree bit for bit, checked in
test_generator_device_matches_host). No oracle input or expected value comes
from the HIP library.

Error measure (per block -- one (sequence, head) slice of o, one 128x128
state, one snapshot): max |x - r| / max |r|, normwise because elementwise
relative error is undefined near zeros. The bar is 2e-3 (fp32 state, bf16
q/k/v inputs).
"""
import os
import sys

import numpy as np

import oracle
import synth

TOL = 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def block_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(x)))
    return float(np.max(np.abs(x - ref)) / den)


def oracle_prefill_unit(seed, H, tok0, L, h, S0=None, scale=1.0, snap_interval=0, snap_slots=0, block=65536,
                        qkv_dtype=synth.BF16, want_o=True, tids=(synth.T_Q, synth.T_K, synth.T_V, synth.T_GK,
                                                               synth.T_BETA)):
    """Oracle over tokens [tok0, tok0+L) of head h of a packed [T, H, 128] batch, fed in blocks.

    Returns (o [L,128] or None, S_end [128,128], snaps or None, n_snapshots)."""
    S = np.zeros((128, 128)) if S0 is None else np.array(S0, dtype=np.float64)
    snaps = np.zeros((snap_slots, 128, 128)) if snap_interval > 0 else None
    outs = []
    cnt = 0
    for p0 in range(0, L, block):
        nb = min(block, L - p0)
        q, k, v, gk, beta = synth.prefill_rows(seed, H, tok0 + p0, nb, h=h, qkv_dtype=qkv_dtype, tids=tids)
        o, S, snaps, c = oracle.recurrent(q, k, v, gk, beta, S, scale=scale, want_o=want_o, pos0=p0,
                                          snap_interval=snap_interval, snap_slots=snap_slots, snaps=snaps)
        cnt += c
        if want_o:
            outs.append(o)
    o = np.concatenate(outs) if (want_o and outs) else (np.zeros((0, 128)) if want_o else None)
    return o, S, snaps, cnt


def threads():
    return min(16, os.cpu_count() or 1)
