"""Checks of the seeded input generator (CPU only)."""
import ctypes
import math

import numpy as np
import pytest
import torch

import synth


def test_philox_known_answers():
    # Known-answer vectors of Philox-4x32-10 (Random123 distribution, SC'11 paper's generator)
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert list(synth.philox4x32_10(ctr, key)) == want


def test_bf16_rne_matches_fp32_path_on_fp32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-30,
                        rng.standard_normal(2000) * 1e30, [0.0, -0.0, 1.0, -2.5]])
    x32 = x.astype(np.float32)  # exactly representable in fp32, so one RNE step
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = synth.round_bf16(x32.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_rne_direct_from_fp64_ties_and_subnormals():
    one = 1.0
    q = 2.0 ** -7  # bf16 spacing at [1, 2)
    cases = {
        one + q / 2: 0x3F80,                 # exact tie -> even (down)
        one + 3 * q / 2: 0x3F82,             # exact tie -> even (up)
        one + q / 2 + 2.0 ** -40: 0x3F81,    # above the tie: up (an fp32 pre-round would tie down)
        one + q / 2 - 2.0 ** -40: 0x3F80,
        2.0 ** -130: 0x0008,                 # bf16 subnormal
        2.0 ** -126: 0x0080,                 # smallest normal
        3.0e38: 0x7F62,
        3.4e38: 0x7F80,                      # past the largest finite bf16 -> inf
        -1.5: 0xBFC0,
    }
    got = synth.round_bf16(np.array(list(cases.keys())))
    assert [int(g) for g in got] == list(cases.values())
    h = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    h = h[((h >> 7) & 0xFF) != 0xFF]  # finite patterns
    assert np.array_equal(synth.round_bf16(synth.bf16_to_f64(h)), h)  # round trip


def test_transcendental_core_accuracy():
    L = synth.lib()
    for f in ("synth_log", "synth_exp", "synth_sqrt", "synth_log1p01"):
        getattr(L, f).argtypes = [ctypes.c_double]
        getattr(L, f).restype = ctypes.c_double
    L.synth_sincos_2pi.argtypes = [ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
    rng = np.random.default_rng(1)
    for x in np.concatenate([rng.uniform(1e-300, 1, 500), [1.0, 0.5, 1e-300]]):
        assert abs(L.synth_log(x) - math.log(x)) <= 4e-16 * max(1.0, abs(math.log(x)))
    for x in rng.uniform(-700, 700, 500):
        assert abs(L.synth_exp(x) - math.exp(x)) <= 4e-16 * math.exp(x)
    for x in rng.uniform(0, 1e12, 500):
        assert abs(L.synth_sqrt(x) - math.sqrt(x)) <= 3e-16 * math.sqrt(x)
    for x in rng.uniform(0, 1, 500):
        assert abs(L.synth_log1p01(x) - math.log1p(x)) <= 5e-16 * max(1e-300, math.log1p(x))
    s, c = ctypes.c_double(), ctypes.c_double()
    for u in np.concatenate([rng.uniform(0, 1, 500), [0.0, 0.125, 0.25, 0.5, 0.75]]):
        L.synth_sincos_2pi(u, ctypes.byref(s), ctypes.byref(c))
        assert abs(s.value - math.sin(2 * math.pi * u)) < 1e-15
        assert abs(c.value - math.cos(2 * math.pi * u)) < 1e-15


def test_determinism_and_slices():
    a = synth.rows(5, synth.T_Q, 0, synth.UNIT_ROW, synth.BF16, 0, 1, 300)
    b = synth.rows(5, synth.T_Q, 0, synth.UNIT_ROW, synth.BF16, 0, 1, 300)
    assert np.array_equal(a, b)
    # one head of a [T, H, 128] tensor regenerated alone equals the slice of the whole
    T, H = 40, 6
    full = synth.prefill_rows(9, H, 0, T)
    for h in (0, 5):
        part = synth.prefill_rows(9, H, 3, 30, h=h)
        for x, y in zip(full, part):
            assert np.array_equal(x[3:33, h], y)
    other = synth.rows(6, synth.T_Q, 0, synth.UNIT_ROW, synth.BF16, 0, 1, 300)
    assert not np.array_equal(a, other)


def test_distributions():
    z = synth.rows(11, 1, 0, synth.NORMAL, synth.F64, 0, 1, 4096).ravel()
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n) and abs(z.var() - 1) < 5 * math.sqrt(2 / n)
    assert abs((z ** 4).mean() - 3) < 0.1
    u = synth.rows(11, 2, 0, synth.UNIT_ROW, synth.F64, 0, 1, 100)
    assert np.allclose(np.linalg.norm(u, axis=1), 1.0, atol=1e-15)
    g = synth.rows(11, 3, 0, synth.NEG_SOFTPLUS, synth.F64, 0, 1, 1000).ravel()
    assert g.max() <= 0 and abs(g.mean() + 0.8063) < 0.01  # E[softplus(N(0,1))] ~= 0.806
    b = synth.rows(11, 4, 0, synth.SIGMOID, synth.F64, 0, 1, 100000, row_len=1).ravel()
    assert 0 < b.min() and b.max() < 1 and abs(b.mean() - 0.5) < 0.005


def test_workload_recipes():
    L2 = synth.prefill_lengths("varlen_h96")
    assert len(L2) == 32 and L2.min() >= 64 and L2.max() <= 24576
    big = synth.loguniform_lengths(123, 200000)
    assert abs(big.mean() - (24576 - 64) / math.log(24576 / 64)) < 60  # log-uniform mean
    acc = synth.geometric_accept(3, 200000)
    assert acc.min() >= 1 and acc.max() <= 8
    p = 1 / 2.7
    clipped_mean = sum(min(8, n) * p * (1 - p) ** (n - 1) for n in range(1, 200))
    assert abs(acc.mean() - clipped_mean) < 0.02
    cu = synth.cu_seqlens([3, 0, 5])
    assert cu.tolist() == [0, 3, 3, 8] and cu.dtype == np.int32
