"""Host-side checks of libkda: it loads, exports every entry point include/kda.h
declares, builds longest-first plans, and rejects bad arguments with
KDA_ERR_INVALID_ARG / KDA_ERR_UNSUPPORTED before touching a device.

Every call below fails validation on the host, so none launches a kernel
(these tests also run safely on a GPU machine).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import linear_attention_recurrence_amd as kda
from linear_attention_recurrence_amd import kda as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call here fails validation first


def declared_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 11
    L = kda.lib()
    for n in names:
        assert hasattr(L, n), f"libkda.so does not export {n}"
    assert set(names) == set(K.EXPORTS)
    assert kda.kda_abi_version() == 4


def test_plan_destroy_and_release():
    """kda_plan_destroy returns a status (NULL is a no-op) and never needs the device; kda_host_release
    with nothing queued (or the buffers of plans destroyed here, pageable without a device) is OK."""
    L = kda.lib()
    assert L.kda_plan_destroy(None) == K.KDA_OK
    plans = [kda.kda_plan_create([0, 40, 75], n_heads=2) for _ in range(3)]
    plans[0].close()
    plans[0].close()  # a second close is a no-op
    with plans[1] as p:
        assert kda.kda_plan_num_items(p) == 4
    assert plans[1].handle is None
    del plans
    kda.kda_host_release()


def test_noalloc_prefill_rejects_oversize_plan():
    """A work list longer than the static scratch (65,520 items) is refused before any device call."""
    cu = np.array([0, 0], dtype=np.int32)
    with kda.kda_plan_create(cu, n_heads=65535) as p:
        assert kda.kda_plan_workspace_bytes(p) > kda.KDA_NOALLOC_SCRATCH_BYTES
        ins = K._Inputs()
        rc = kda.lib().kda_chunk_prefill_noalloc(p.handle, ctypes.byref(ins), None, ctypes.c_void_p(16), None, None, 0,
                                                 None, 1.0, None)
        assert rc == K.KDA_ERR_INVALID_ARG
        assert "static scratch" in kda.kda_last_error()
    with kda.kda_plan_create(cu, n_heads=65520) as p:
        assert kda.kda_plan_workspace_bytes(p) == kda.KDA_NOALLOC_SCRATCH_BYTES


def test_plan_lpt_order_and_ties():
    cu = [0, 5, 100, 100, 140, 235]  # lengths 5, 95, 0, 40, 95
    p = kda.kda_plan_create(cu, n_heads=3)
    it = kda.kda_plan_items(p)
    lens = it[:, 3]
    assert list(lens) == sorted(lens, reverse=True)
    # equal lengths keep (sequence, head) ascending
    top = [tuple(x[:2]) for x in it if x[3] == 95]
    assert top == [(1, 0), (1, 1), (1, 2), (4, 0), (4, 1), (4, 2)]
    for n, h, t0, L in it:
        assert t0 == cu[n] and L == cu[n + 1] - cu[n] and 0 <= h < 3
    assert kda.kda_plan_workspace_bytes(p) == 256 + 16 * 15
    fifo = kda.kda_plan_items(kda.kda_plan_create(cu, n_heads=3, order=kda.KDA_PLAN_FIFO))
    assert [tuple(x[:2]) for x in fifo] == [(n, h) for n in range(5) for h in range(3)]


def test_plan_value_blocks():
    cu = [0, 5, 100, 100, 140, 235]  # lengths 5, 95, 0, 40, 95
    p = kda.kda_plan_create(cu, n_heads=3, v_blocks=2)
    assert kda.kda_plan_v_blocks(p) == 2 and kda.kda_plan_num_items(p) == 30
    assert kda.kda_plan_workspace_bytes(p) == 256 + 16 * 30
    it = kda.kda_plan_items(p)
    h, vb = it[:, 1] & 0xffff, it[:, 1] >> 16
    assert list(it[:, 3]) == sorted(it[:, 3], reverse=True)
    # equal lengths keep (sequence, head, value block) ascending; every triple appears once
    top = [(int(a), int(b), int(c)) for a, b, c, L in zip(it[:, 0], h, vb, it[:, 3]) if L == 95]
    assert top == [(n, hh, v) for n in (1, 4) for hh in range(3) for v in range(2)]
    assert sorted(zip(it[:, 0], h, vb)) == [(n, hh, v) for n in range(5) for hh in range(3) for v in range(2)]
    fifo = kda.kda_plan_items(kda.kda_plan_create(cu, n_heads=3, order=kda.KDA_PLAN_FIFO, v_blocks=2))
    assert [(x[0], x[1] & 0xffff, x[1] >> 16) for x in fifo] == [(n, hh, v) for n in range(5) for hh in range(3)
                                                                  for v in range(2)]
    # the one-block plan is kda_plan_create's, with a zero value block in every item
    one = kda.kda_plan_items(kda.kda_plan_create(cu, n_heads=3, v_blocks=1))
    assert np.array_equal(one, kda.kda_plan_items(kda.kda_plan_create(cu, n_heads=3)))
    assert np.all(one[:, 1] >> 16 == 0)
    # automatic choice: 1 or 2, never more items than the device could need
    auto = kda.kda_plan_create(cu, n_heads=3, v_blocks=0)
    assert kda.kda_plan_v_blocks(auto) in (1, 2)
    assert kda.kda_plan_v_blocks(kda.kda_plan_create([0, 8] * 1, n_heads=4096, v_blocks=0)) == 1


@pytest.mark.parametrize("cu,H,iv,vb,msg", [
    ([1, 5], 1, 0, 1, "cu_seqlens[0]"),
    ([0, 5, 3], 1, 0, 1, "non-decreasing"),
    ([0, 5], 0, 0, 1, "n_heads"),
    ([0, 5], 1, 48, 1, "multiple"),
    ([0, 5], 1, -32, 1, "multiple"),
    ([0, 5], 1, 0, 3, "v_blocks"),
    ([0, 5], 1, 0, -1, "v_blocks"),
    ([0, 5], 65536, 0, 1, "65535"),
])
def test_plan_rejects(cu, H, iv, vb, msg):
    with pytest.raises(kda.KdaError) as e:
        kda.kda_plan_create(cu, n_heads=H, snap_interval=iv, v_blocks=vb)
    assert e.value.status == kda.KDA_ERR_INVALID_ARG and msg in str(e.value)


def _inputs():
    return K._Inputs(FAKE.value, FAKE.value + 0x100000, FAKE.value + 0x200000, FAKE.value + 0x300000,
                     FAKE.value + 0x400000)


def test_prefill_rejects_bad_arguments():
    L = kda.lib()
    p = kda.kda_plan_create([0, 64], n_heads=1, snap_interval=32)
    ins = _inputs()
    ws = ctypes.c_void_p(0x9000000)
    out = ctypes.c_void_p(0x8000000)
    o = ctypes.c_void_p(0xA000000)
    # NULL plan, inputs, state_out, workspace
    assert L.kda_chunk_prefill(None, ctypes.byref(ins), None, out, o, None, 0, None, ws, 1.0, 0, None) == 1
    assert L.kda_chunk_prefill(p.handle, None, None, out, o, None, 0, None, ws, 1.0, 0, None) == 1
    assert L.kda_chunk_prefill(p.handle, ctypes.byref(ins), None, None, o, None, 0, None, ws, 1.0, 0, None) == 1
    assert L.kda_chunk_prefill(p.handle, ctypes.byref(ins), None, out, o, None, 0, None, None, 1.0, 0, None) == 1
    # o overlapping q
    assert L.kda_chunk_prefill(p.handle, ctypes.byref(ins), None, out, FAKE, None, 0, None, ws, 1.0, 0, None) == 1
    assert "o overlaps" in kda.kda_last_error()
    # snapshots requested with zero slots
    assert L.kda_chunk_prefill(p.handle, ctypes.byref(ins), None, out, o, ctypes.c_void_p(0xB000000), 0, None, ws,
                               1.0, 0, None) == 1
    assert "snap_slots" in kda.kda_last_error()
    # partial overlap of state_in and state_out
    assert L.kda_chunk_prefill(p.handle, ctypes.byref(ins), ctypes.c_void_p(0x8000000 + 4096), out, o, None, 0,
                               None, ws, 1.0, 0, None) == 1
    assert "state_in and state_out" in kda.kda_last_error()
    # unknown flag bits
    assert L.kda_chunk_prefill(p.handle, ctypes.byref(ins), None, out, o, None, 0, None, ws, 1.0, 2, None) == 1


def _ring(length, base=0xC000000):
    return K._Ring(base, base + 0x1000000, base + 0x2000000, base + 0x3000000, length)


def test_verify_rejects_bad_arguments():
    L = kda.lib()
    ins = _inputs()
    pool, slots, o = ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x30000000), ctypes.c_void_p(0x40000000)
    args = lambda **kw: dict(dict(B=2, T=8, H=2, Lyr=3, layer=0, S=4, dt=kda.KDA_BF16, ring=None), **kw)

    def call(B=2, T=8, H=2, Lyr=3, layer=0, S=4, dt=kda.KDA_BF16, ring=None, commit_len=None, commit_pool=None,
             o_=o):
        r = ctypes.byref(ring) if ring is not None else None
        return L.kda_verify(B, T, H, Lyr, layer, S, dt, ctypes.byref(ins), pool, slots, o_, r, None, commit_len,
                            commit_pool, 1.0, None)

    assert call(T=0) == 1
    assert call(layer=3) == 1
    assert call(layer=-1) == 1
    assert call(S=0) == 1
    assert call(dt=7) == 1
    assert call(dt=kda.KDA_F32, ring=_ring(16)) == 2  # fp32 inputs cannot be recorded in the bf16 ring
    assert call(ring=_ring(12)) == 1  # not a power of two
    assert call(ring=_ring(8)) == 1   # < 2 * n_tok
    assert "power of two" in kda.kda_last_error()
    assert call(commit_len=FAKE) == 1  # commit_len without commit_pool
    assert call(commit_len=ctypes.c_void_p(0x50000000), commit_pool=ctypes.c_void_p(0x20000000 + 65536)) == 1
    assert call(o_=ctypes.c_void_p(0x20000000)) == 1  # o overlaps the state pool
    assert call(B=0) == 0  # nothing to do


def test_fold_rejects_bad_arguments():
    L = kda.lib()
    pool, slots, acc = ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x30000000), ctypes.c_void_p(0x31000000)
    r16 = _ring(16)
    assert L.kda_replay_fold(2, 2, 3, 4, pool, slots, None, None, acc, None) == 1
    assert L.kda_replay_fold(2, 2, 3, 4, pool, slots, ctypes.byref(_ring(6)), None, acc, None) == 1
    assert L.kda_replay_fold(2, 2, 3, 4, pool, None, ctypes.byref(r16), None, acc, None) == 1
    assert L.kda_replay_fold(2, 2, 3, 4, pool, slots, ctypes.byref(r16), None, None, None) == 1
    assert L.kda_replay_fold(2, 0, 3, 4, pool, slots, ctypes.byref(r16), None, acc, None) == 1
    # state pool overlapping the ring
    assert L.kda_replay_fold(2, 2, 3, 4, ctypes.c_void_p(0xC000000), slots, ctypes.byref(r16), None, acc, None) == 1
    assert L.kda_replay_fold(0, 2, 3, 4, pool, slots, ctypes.byref(r16), None, acc, None) == 0


def test_fold_verify_rejects_bad_arguments():
    L = kda.lib()
    ins = _inputs()
    pool, slots, o = ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x30000000), ctypes.c_void_p(0x40000000)
    flen = ctypes.c_void_p(0x31000000)

    def call(B=2, T=8, H=2, Lyr=3, layer=0, S=4, ring=_ring(16), fold_len=flen, o_=o, pool_=pool):
        r = ctypes.byref(ring) if ring is not None else None
        return L.kda_fold_verify(B, T, H, Lyr, layer, S, ctypes.byref(ins), pool_, slots, o_, r, None, fold_len, None,
                                 1.0, None)

    assert call(T=0) == 1
    assert call(layer=3) == 1
    assert call(ring=None) == 1                     # the ring is required
    assert call(fold_len=None) == 1                 # so are the fold lengths
    assert call(ring=_ring(12)) == 1                # not a power of two
    assert call(T=4, ring=_ring(4)) == 1            # < 2 * n_tok
    assert call(T=9, ring=_ring(32)) == 2           # more than 8 draft tokens
    assert call(T=4, ring=_ring(32)) == 2           # a ring longer than 16 (folds of more than 8 entries)
    assert "16" in kda.kda_last_error()
    assert call(o_=ctypes.c_void_p(0x20000000)) == 1  # o overlaps the state pool
    assert call(pool_=ctypes.c_void_p(0xC000000)) == 1  # the pool overlaps the ring
    assert call(B=0) == 0                           # nothing to do


def test_verify_ragged_rejects_bad_arguments():
    L = kda.lib()
    ins = _inputs()
    pool, slots, o = ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x30000000), ctypes.c_void_p(0x40000000)
    cu = ctypes.c_void_p(0x31000000)

    def call(B=2, max_tok=8, total=10, H=2, Lyr=3, layer=0, S=4, ring=_ring(16), cu_=cu, o_=o):
        r = ctypes.byref(ring) if ring is not None else None
        return L.kda_verify_ragged(B, max_tok, total, H, Lyr, layer, S, ctypes.byref(ins), cu_, pool, slots, o_, r,
                                   None, 1.0, None)

    assert call(max_tok=0) == 1
    assert call(max_tok=17, ring=_ring(64)) == 1    # windows of at most 16 tokens
    assert call(total=-1) == 1
    assert call(B=-1) == 1
    assert call(layer=3) == 1
    assert call(cu_=None) == 1                      # the window bounds are required
    assert call(ring=_ring(12)) == 1                # not a power of two
    assert call(max_tok=16, ring=_ring(16)) == 1    # < 2 * max_tok
    assert call(o_=ctypes.c_void_p(0x20000000)) == 1  # o overlaps the state pool
    assert call(o_=ctypes.c_void_p(0x31000000)) == 1  # o overlaps cu_tok
    assert call(o_=ctypes.c_void_p(0xC000000)) == 1   # o overlaps the ring
    assert call(B=0) == 0                           # nothing to do
    assert call(total=0) == 0                       # every window is empty


def test_gated_rejects_bad_arguments():
    L = kda.lib()
    o, g, w, y = (ctypes.c_void_p(x) for x in (0x20000000, 0x30000000, 0x31000000, 0x40000000))
    norm = lambda rows=16, eps=1e-6, o_=o, y_=y: L.kda_gated_rmsnorm(rows, o_, g, w, eps, y_, None)
    assert norm(rows=-1) == 1
    assert norm(eps=-1.0) == 1
    assert norm(eps=float("inf")) == 1
    assert norm(o_=None) == 1
    assert norm(y_=ctypes.c_void_p(0x20000000 + 64)) == 1  # y overlaps o
    assert norm(rows=0) == 0                                # nothing to do
    ins = _inputs()
    ws, st = ctypes.c_void_p(0x50000000), ctypes.c_void_p(0x60000000)
    p1 = kda.kda_plan_create([0, 64, 100], n_heads=2)
    p2 = kda.kda_plan_create([0, 64, 100], n_heads=2, v_blocks=2)

    def pre(plan=p1, gate=g, eps=1e-6, y_=y):
        return L.kda_chunk_prefill_gated(plan.handle, ctypes.byref(ins), gate, w, eps, None, st, y_, None, 0, None,
                                         ws, 1.0, 0, None)

    assert pre(y_=None) == 1
    assert pre(gate=None) == 1
    assert pre(eps=-0.5) == 1
    assert pre(plan=p2) == 2                                # half-row items cannot normalise a row
    assert "value block" in kda.kda_last_error()
    assert pre(y_=ctypes.c_void_p(0x30000000)) == 1         # y overlaps the gate
    assert pre(y_=ctypes.c_void_p(0x60000000)) == 1         # y overlaps state_out


def test_prologue_rejects_bad_arguments():
    L = kda.lib()
    P = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(13)]
    cu, xq, xk, xv, w, sin, sout, b, g, q, k, v, beta = P
    gk = ctypes.c_void_p(0xE0000000)

    def call(N=2, T=10, H=2, W=4, eps=1e-6, sin_=sin, sout_=sout, q_=q, cu_=cu):
        return L.kda_prologue(N, T, H, W, cu_, xq, xk, xv, w, sin_, sout_, b, g, eps, q_, k, v, beta, gk, None)

    assert call(W=0) == 1 and call(W=9) == 1      # conv width 1..8
    assert call(H=0) == 1 and call(T=-1) == 1 and call(H=70000) == 1
    assert call(N=1 << 30, H=60000, W=8) == 1                # the carried state's grid would overflow
    assert call(N=0) == 1                          # tokens without sequences
    assert call(eps=-1.0) == 1
    assert call(cu_=None) == 1
    assert call(q_=None) == 1
    assert call(sout_=ctypes.c_void_p(0x60000000 + 16)) == 1  # the carried state is not updated in place
    assert call(q_=ctypes.c_void_p(0xA0000000 + 8)) == 1      # row buffers are 16-byte aligned
    assert call(q_=ctypes.c_void_p(0x20000000)) == 1          # q overlaps xq
    assert call(N=0, T=0) == 0                                # nothing to do


def test_state_move_rejects_bad_arguments():
    L = kda.lib()
    pool = ctypes.c_void_p(0x40000000)
    moves = ctypes.c_void_p(0x80000000)

    def call(n=3, mv=moves, S=4, sf=16384, pl=pool):
        return L.kda_state_move(n, mv, S, sf, pl, None)

    assert call(n=-1) == 1 and call(S=0) == 1
    assert call(sf=0) == 1 and call(sf=6) == 1                  # a positive multiple of 4 floats
    assert call(mv=None) == 1 and call(pl=None) == 1
    assert call(pl=ctypes.c_void_p(0x40000000 + 4)) == 1         # 16-byte aligned pool
    assert call(mv=ctypes.c_void_p(0x40000000 + 64)) == 1        # the move list inside the pool
    assert call(S=2, sf=1 << 62) == 1                            # size overflow
    assert call(n=0, mv=None, pl=None) == 0                      # nothing to do


def test_decode_rejects_bad_arguments():
    L = kda.lib()
    P = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(14)]
    xq, xk, xv, w, cs, b, g, pool, slots, gate, nw, y, o, _ = P

    def call(B=2, H=4, Lyr=3, layer=1, S=5, W=4, cs_=cs, y_=y, eps=1e-6, scale=1.0):
        return L.kda_decode(B, H, Lyr, layer, S, W, xq, xk, xv, w, cs_, b, g, pool, slots, gate, nw, eps, eps, scale,
                            y_, o, None)

    assert call(W=0) == 1 and call(W=9) == 1 and call(layer=3) == 1 and call(H=70000) == 1
    assert call(eps=-1.0) == 1 and call(scale=float("inf")) == 1
    assert call(cs_=None) == 1                                  # the conv state is required for W > 1
    assert call(y_=ctypes.c_void_p(0x10000000 + 16)) == 1       # y overlaps xq
    assert call(y_=ctypes.c_void_p(0xC0000000 + 8)) == 1        # not 16-byte aligned
    assert call(B=0) == 0                                       # nothing to do


def test_state_move_binding_empty_and_shapes():
    import torch

    pool = torch.zeros((2, 4))
    kda.kda_state_move(pool, torch.tensor([], dtype=torch.int32))  # an empty move list is a no-op
    with pytest.raises(ValueError):
        kda.kda_state_move(pool, torch.zeros((3,), dtype=torch.int32))  # not [n, 2]


def test_binding_checks_shapes_without_device():
    import torch

    p = kda.kda_plan_create([0, 64], n_heads=1)
    x = torch.zeros((64, 1, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kda.kda_chunk_prefill(p, x, x, x, x.float(), torch.zeros((64, 1)), torch.zeros((1, 1, 128, 128)),
                              torch.zeros((64, 1, 128)), torch.zeros(kda.kda_plan_workspace_bytes(p), dtype=torch.uint8))


def test_probes_reject_bad_arguments():
    """The measurement probes refuse bad sizes, alignment and overlap before any device call."""
    L = kda.lib()
    p16, p32 = ctypes.c_void_p(16), ctypes.c_void_p(32)
    flop = ctypes.c_int64(0)
    cases = [
        L.kda_probe_copy(None, p32, 16, None),
        L.kda_probe_copy(p16, p32, 15, None),     # not a multiple of 16
        L.kda_probe_copy(ctypes.c_void_p(17), p32, 16, None),  # misaligned
        L.kda_probe_copy(p16, p32, 32, None),     # overlapping
        L.kda_probe_read(p16, 0, p32, 256, None),
        L.kda_probe_read(p16, 16, p32, 255, None),  # sink too small for one workgroup
        L.kda_probe_mfma(0, 1.0, p32, 256, ctypes.byref(flop), None),
        L.kda_probe_mfma(1, 1.0, p32, 100, ctypes.byref(flop), None),
        L.kda_probe_mfma(1, 1.0, p32, 256, None, None),
    ]
    assert all(rc == K.KDA_ERR_INVALID_ARG for rc in cases), cases
