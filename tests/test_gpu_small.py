"""GPU parity on small shapes that still span several chunks, ragged tails and
every edge case; all calls go through the C ABI (libkda.so)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.gpu as sg
import linear_attention_recurrence_amd as kda
from kda_ref import TOL, block_err, log, oracle_prefill_unit

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def np_(t):
    return t.detach().cpu().numpy()


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


# ---------------------------------------------------------------- generator
@pytest.mark.parametrize("kind,dtype,row_len", [
    (synth.NORMAL, torch.float32, 128), (synth.NORMAL, torch.bfloat16, 128), (synth.UNIT_ROW, torch.bfloat16, 128),
    (synth.UNIT_ROW, torch.float32, 128), (synth.NEG_SOFTPLUS, torch.float32, 128), (synth.SIGMOID, torch.float32, 1),
    (synth.NORMAL, torch.float64, 128)])
def test_generator_device_matches_host(gpu, kind, dtype, row_len):
    log(f"generator kind={kind} dtype={dtype}")
    n_rows, start, step = 3000, 17, 3
    t = torch.empty(n_rows * row_len, dtype=dtype, device=DEV)
    sg.fill(t, 77, 5, 2, kind, row_start=start, row_step=step, row_len=row_len, scale=0.3)
    hd = {torch.float32: synth.F32, torch.bfloat16: synth.BF16, torch.float64: synth.F64}[dtype]
    h = synth.rows(77, 5, 2, kind, hd, start, step, n_rows, row_len, 0.3).ravel()
    if dtype == torch.bfloat16:
        assert np.array_equal(bits(t).view(np.uint16), h)
    else:
        assert np.array_equal(np_(t).view(np.uint64 if dtype == torch.float64 else np.uint32),
                              h.view(np.uint64 if dtype == torch.float64 else np.uint32))


# ---------------------------------------------------------------- verify and fold
def make_verify_case(seed, B, T, H, L, S, R):
    g = torch.Generator().manual_seed(seed)
    slot_idx = torch.randperm(S, generator=g)[:B].to(torch.int32)
    pool = sg.states(seed, S * L * H, DEV).view(S, L, H, 128, 128)
    ins = [sg.prefill_inputs(seed, B * T, H, DEV, sub=l) for l in range(L)]
    ring_start = torch.randint(0, 4 * R, (B,), generator=g, dtype=torch.int32)
    return slot_idx, pool, ins, ring_start


def host_inputs(seed, B, T, H, l, b, h):
    q, k, v, gk, beta = synth.prefill_rows(seed, H, b * T, T, h=h, sub=l)
    return q, k, v, gk, beta


def test_verify_and_fold_small(gpu):
    seed, B, T, H, L, S, R = 31, 3, 5, 2, 2, 6, 16
    log("verify/fold small")
    slot_idx, pool, ins, ring_start = make_verify_case(seed, B, T, H, L, S, R)
    commit_len = torch.tensor([2, 5, 0], dtype=torch.int32)
    pool0 = pool.clone()
    ring = kda.Ring.empty(S, L, H, R, DEV)
    for buf in (ring.k, ring.v):
        buf.view(torch.int16).fill_(0x7FC1)  # sentinel bit pattern
    ring.gk.fill_(-7.0)
    ring.beta.fill_(-7.0)
    commit = torch.full_like(pool, -3.0)
    outs = []
    for l in range(L):
        q, k, v, gk, beta = ins[l]
        o = torch.empty((B * T, H, 128), device=DEV)
        kda.kda_verify(q, k, v, gk, beta, pool, slot_idx.to(DEV), o, layer=l, n_tok=T, ring=ring,
                       ring_start=ring_start.to(DEV), commit_len=commit_len.to(DEV), commit_pool=commit, scale=0.6)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool0), "verify wrote the committed state"
    rb = {n: np_(x) if x.dtype != torch.bfloat16 else bits(x).view(np.uint16)
          for n, x in (("k", ring.k), ("v", ring.v), ("gk", ring.gk), ("beta", ring.beta))}
    worst = 0.0
    for l in range(L):
        o = np_(outs[l]).reshape(B, T, H, 128)
        for b in range(B):
            s = int(slot_idx[b])
            for h in range(H):
                q, k, v, gk, beta = host_inputs(seed, B, T, H, l, b, h)
                S0 = np_(pool0[s, l, h])
                c = int(commit_len[b])
                o_ref, Sc_ref, _ = oracle.verify(q, k, v, gk, beta, S0, scale=0.6, commit_len=c)
                worst = max(worst, block_err(o[b, :, h], o_ref))
                if c > 0:
                    worst = max(worst, block_err(np_(commit[s, l, h]), Sc_ref))
                # the ring holds the raw inputs, bit for bit, at (start + t) & (R - 1); other slots untouched
                pos = [(int(ring_start[b]) + t) & (R - 1) for t in range(T)]
                assert np.array_equal(rb["k"][s, l, h, pos], k) and np.array_equal(rb["v"][s, l, h, pos], v)
                assert np.array_equal(rb["gk"][s, l, h, pos], gk) and np.array_equal(rb["beta"][s, l, h, pos], beta)
                other = [p for p in range(R) if p not in pos]
                assert np.all(rb["gk"][s, l, h, other] == -7.0)
    unused = [s for s in range(S) if s not in slot_idx.tolist()]
    assert torch.all(commit[unused] == -3.0)
    b0 = int((commit_len == 0).nonzero()[0])
    assert torch.all(commit[int(slot_idx[b0])] == -3.0), "commit_len 0 must not write"
    log(f"verify small worst err {worst:.2e}")
    assert worst <= TOL

    # fold with the same accepted lengths == verify's commit, bit for bit
    acc = commit_len.clone()
    folded = pool0.clone()
    # poison every ring entry past the accepted prefix: the fold must never read it
    for b in range(B):
        s = int(slot_idx[b])
        for t in range(int(acc[b]), R):
            p = (int(ring_start[b]) + t) & (R - 1)
            ring.gk[s, :, :, p] = float("nan")
            ring.beta[s, :, :, p] = float("nan")
    kda.kda_replay_fold(folded, slot_idx.to(DEV), ring, acc.to(DEV), ring_start=ring_start.to(DEV))
    torch.cuda.synchronize()
    for b in range(B):
        s = int(slot_idx[b])
        if int(acc[b]) > 0:
            assert torch.equal(folded[s], commit[s]), f"fold differs from verify commit for request {b}"
        else:
            assert torch.equal(folded[s], pool0[s])
    for s in range(S):
        if s not in slot_idx.tolist():
            assert torch.equal(folded[s], pool0[s])


@pytest.mark.parametrize("T,R,B,H", [(8, 16, 6, 2), (5, 16, 6, 2), (1, 2, 6, 2), (3, 8, 6, 2), (8, 16, 5, 3)])
def test_fold_verify_bitwise(gpu, T, R, B, H):
    """kda_fold_verify == kda_replay_fold of the previous window, then kda_verify of the new one, bit for
    bit: the folded pool (every layer, every slot), o, and the ring (the previous window untouched, the new
    entries written); fold lengths 0 .. R/2 (0 must not write), an invalid slot, windows that wrap, and an
    odd number of (request, head) units (a workgroup's second half then has no unit of its own)."""
    seed, L, S = 41, 3, 8
    g = torch.Generator().manual_seed(seed + T)
    slot_idx = torch.randperm(S, generator=g)[:B].to(torch.int32)
    slot_idx[3] = -1
    pool0 = sg.states(seed, S * L * H, DEV).view(S, L, H, 128, 128)
    ring = kda.Ring.empty(S, L, H, R, DEV)
    fold_start = torch.randint(0, 4 * R, (B,), generator=g, dtype=torch.int32)
    prev_T = R // 2
    # the previous window: a verify of prev_T tokens recorded at fold_start
    prev = [sg.prefill_inputs(seed + 1, B * prev_T, H, DEV, sub=l) for l in range(L)]
    scratch_o = torch.empty((B * prev_T, H, 128), device=DEV)
    for l in range(L):
        kda.kda_verify(*prev[l], pool0, slot_idx.to(DEV), scratch_o, layer=l, n_tok=prev_T, ring=ring,
                       ring_start=fold_start.to(DEV))
    fold_len = torch.tensor([prev_T, 0, 1, 2, prev_T - 1 if prev_T > 1 else 0, 3 % (prev_T + 1)][:B], dtype=torch.int32)
    ring_start = fold_start + prev_T  # the next window starts where the previous one ended
    ins = [sg.prefill_inputs(seed + 2, B * T, H, DEV, sub=l) for l in range(L)]
    # reference: fold, then verify from the folded pool
    ref_pool = pool0.clone()
    ref_ring = kda.Ring(ring.k.clone(), ring.v.clone(), ring.gk.clone(), ring.beta.clone())
    kda.kda_replay_fold(ref_pool, slot_idx.to(DEV), ref_ring, fold_len.to(DEV), ring_start=fold_start.to(DEV))
    ref_o = []
    for l in range(L):
        o = torch.full((B * T, H, 128), -9.0, device=DEV)
        kda.kda_verify(*ins[l], ref_pool, slot_idx.to(DEV), o, layer=l, n_tok=T, ring=ref_ring,
                       ring_start=ring_start.to(DEV), scale=0.7)
        ref_o.append(o)
    # fused, one layer at a time
    pool = pool0.clone()
    fus_o = []
    for l in range(L):
        o = torch.full((B * T, H, 128), -9.0, device=DEV)
        kda.kda_fold_verify(*ins[l], pool, slot_idx.to(DEV), o, layer=l, n_tok=T, ring=ring, fold_len=fold_len.to(DEV),
                            fold_start=fold_start.to(DEV), ring_start=ring_start.to(DEV), scale=0.7)
        fus_o.append(o)
    torch.cuda.synchronize()
    log(f"fold_verify T={T} R={R}: fold lengths {fold_len.tolist()}, slots {slot_idx.tolist()}")
    assert torch.equal(pool, ref_pool)
    for l in range(L):
        assert torch.equal(fus_o[l], ref_o[l])
    for a, b in ((ring.k, ref_ring.k), (ring.v, ref_ring.v), (ring.gk, ref_ring.gk), (ring.beta, ref_ring.beta)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    # the invalid slot's request wrote nothing; fold length 0 left its state as it was
    assert torch.all(fus_o[0].view(B, T, H, 128)[3] == -9.0)
    s1 = int(slot_idx[1])
    assert torch.equal(pool[s1], pool0[s1])


@pytest.mark.parametrize("T,use_ring,H", [(1, True, 2), (5, True, 2), (8, True, 2), (16, True, 2), (8, False, 2),
                                           (17, True, 2), (8, True, 3), (16, True, 3)])
def test_verify_without_commit(gpu, T, use_ring, H):
    """The call shape of a speculative step (no recurrent commit): up to 16 tokens take the chunked
    matrix-core path, longer windows the token-by-token kernel; either way the outputs match the
    oracle, the ring holds the raw inputs bit for bit and the committed state is untouched. H = 3 makes
    the number of (request, head) units odd."""
    seed, B, L, S = 41 + T, 3, 2, 6
    R = 32 if T <= 16 else 64
    log(f"verify without commit T={T} ring={use_ring} H={H}")
    slot_idx, pool, ins, ring_start = make_verify_case(seed, B, T, H, L, S, R)
    slot_idx[1] = -1  # a request with no slot: skipped, its outputs stay as they were
    pool0 = pool.clone()
    ring = kda.Ring.empty(S, L, H, R, DEV) if use_ring else None
    if ring is not None:
        ring.gk.fill_(-7.0)
    worst = 0.0
    for l in range(L):
        q, k, v, gk, beta = ins[l]
        o = torch.full((B * T, H, 128), -9.0, device=DEV)
        kda.kda_verify(q, k, v, gk, beta, pool, slot_idx.to(DEV), o, layer=l, n_tok=T, ring=ring,
                       ring_start=ring_start.to(DEV) if use_ring else None, scale=0.6)
        torch.cuda.synchronize()
        on = np_(o).reshape(B, T, H, 128)
        for b in range(B):
            s = int(slot_idx[b])
            if s < 0:
                assert np.all(on[b] == -9.0)
                continue
            for h in range(H):
                q_, k_, v_, gk_, beta_ = host_inputs(seed, B, T, H, l, b, h)
                o_ref, _, _ = oracle.verify(q_, k_, v_, gk_, beta_, np_(pool0[s, l, h]), scale=0.6)
                worst = max(worst, block_err(on[b, :, h], o_ref))
                if ring is not None:
                    pos = [(int(ring_start[b]) + t) & (R - 1) for t in range(T)]
                    assert np.array_equal(bits(ring.k[s, l, h, pos]).view(np.uint16), k_)
                    assert np.array_equal(bits(ring.v[s, l, h, pos]).view(np.uint16), v_)
                    assert np.array_equal(np_(ring.gk[s, l, h, pos]), gk_)
                    assert np.array_equal(np_(ring.beta[s, l, h, pos]), beta_)
    assert torch.equal(pool, pool0), "verify wrote the committed state"
    log(f"verify without commit T={T} worst err {worst:.2e}")
    assert worst <= TOL


def ragged_windows(cu, total, max_tok):
    """The windows kda_verify_ragged reads from cu_tok (clamped as include/kda.h states): (first row, length)."""
    out = []
    for b in range(len(cu) - 1):
        s0 = min(max(int(cu[b]), 0), total)
        e = min(max(int(cu[b + 1]), s0), total)
        out.append((s0, min(e - s0, max_tok)))
    return out


def check_ragged(seed, l, cu, total, max_tok, H, slot_idx, pool0, o, ring, ring0, ring_start, R, scale):
    """o against the oracle on every window, the ring entries bit for bit, and everything outside the
    windows untouched (o rows not in any window, ring positions not written)."""
    worst = 0.0
    on = np_(o)
    covered = np.zeros(total, dtype=bool)
    written = {}
    for b, (first, n) in enumerate(ragged_windows(cu, total, max_tok)):
        s = int(slot_idx[b])
        if n == 0 or s < 0:
            continue
        covered[first:first + n] = True
        for h in range(H):
            q_, k_, v_, gk_, beta_ = synth.prefill_rows(seed, H, first, n, h=h, sub=l)
            o_ref, _, _ = oracle.verify(q_, k_, v_, gk_, beta_, np_(pool0[s, l, h]), scale=scale)
            worst = max(worst, block_err(on[first:first + n, h], o_ref))
            pos = [(int(ring_start[b]) + t) & (R - 1) for t in range(n)]
            written.setdefault((s, h), set()).update(pos)
            assert np.array_equal(bits(ring.k[s, l, h, pos]).view(np.uint16), k_)
            assert np.array_equal(bits(ring.v[s, l, h, pos]).view(np.uint16), v_)
            assert np.array_equal(np_(ring.gk[s, l, h, pos]), gk_)
            assert np.array_equal(np_(ring.beta[s, l, h, pos]), beta_)
    assert np.all(on[~covered] == -9.0), "rows outside every window were written"
    for t_new, t_old in ((ring.k, ring0.k), (ring.v, ring0.v), (ring.gk, ring0.gk), (ring.beta, ring0.beta)):
        a, b_ = bits(t_new[:, l]), bits(t_old[:, l])
        for (s, h), pos in written.items():
            pos = sorted(pos)
            a[s, h, pos] = b_[s, h, pos]
        assert np.array_equal(a, b_), "ring entries outside the windows changed"
    return worst


@pytest.mark.parametrize("max_tok,lens", [(8, [3, 0, 8, 1, 5, 7, 2]), (16, [16, 9, 0, 2, 13, 8, 1]),
                                          (8, [8, 8, 8, 8, 8, 8, 8])])
def test_verify_ragged(gpu, max_tok, lens):
    """Per-request trimmed windows packed back to back: o against the oracle on each window, the ring
    entries bit for bit and nothing else written (empty windows, an invalid slot); o and ring bitwise
    equal to one kda_verify call per request with n_tok = n_b where both take the same padded window;
    all windows full equals a plain kda_verify call bit for bit; the committed state untouched."""
    seed, H, L, S, R = 77 + max_tok + sum(lens), 3, 2, 10, 32
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    g = torch.Generator().manual_seed(seed)
    slot_idx = torch.randperm(S, generator=g)[:B].to(torch.int32)
    slot_idx[3] = -1
    pool = sg.states(seed, S * L * H, DEV).view(S, L, H, 128, 128)
    pool0 = pool.clone()
    ring_start = torch.randint(0, 4 * R, (B,), generator=g, dtype=torch.int32)
    ring = kda.Ring.empty(S, L, H, R, DEV)
    for t in (ring.k, ring.v, ring.gk, ring.beta):
        t.view(torch.int16 if t.element_size() == 2 else torch.int32).fill_(-7)
    ring0 = kda.Ring(ring.k.clone(), ring.v.clone(), ring.gk.clone(), ring.beta.clone())
    ref_ring = kda.Ring(ring.k.clone(), ring.v.clone(), ring.gk.clone(), ring.beta.clone())
    cu_d, slot_d, rs_d = torch.from_numpy(cu).to(DEV), slot_idx.to(DEV), ring_start.to(DEV)
    worst = 0.0
    log(f"ragged verify max_tok={max_tok} lens={lens}")
    for l in range(L):
        ins = sg.prefill_inputs(seed, total, H, DEV, sub=l)
        o = torch.full((total, H, 128), -9.0, device=DEV)
        kda.kda_verify_ragged(*ins, cu_d, pool, slot_d, o, layer=l, max_tok=max_tok, ring=ring, ring_start=rs_d,
                              scale=0.6)
        # the same windows one request at a time through kda_verify
        ref_o = torch.full((total, H, 128), -9.0, device=DEV)
        for b, n in enumerate(lens):
            if n == 0:
                continue
            r0, r1 = int(cu[b]), int(cu[b + 1])
            kda.kda_verify(*(x[r0:r1] for x in ins), pool, slot_d[b:b + 1], ref_o[r0:r1], layer=l, n_tok=n,
                           ring=ref_ring, ring_start=rs_d[b:b + 1], scale=0.6)
        if all(n == max_tok for n in lens):
            full_o = torch.full((total, H, 128), -9.0, device=DEV)
            kda.kda_verify(*ins, pool, slot_d, full_o, layer=l, n_tok=max_tok, scale=0.6)
        torch.cuda.synchronize()
        worst = max(worst, check_ragged(seed, l, cu, total, max_tok, H, slot_idx, pool0, o, ring, ring0, ring_start,
                                        R, 0.6))
        for b, n in enumerate(lens):
            if n and (n > 8) == (max_tok > 8):  # the same padded window (8 or 16 tokens) on both paths
                r0, r1 = int(cu[b]), int(cu[b + 1])
                assert torch.equal(o[r0:r1], ref_o[r0:r1])
        if all(n == max_tok for n in lens):
            assert torch.equal(o, full_o)
    for a, b_ in ((ring.k, ref_ring.k), (ring.v, ref_ring.v), (ring.gk, ref_ring.gk), (ring.beta, ref_ring.beta)):
        assert np.array_equal(bits(a), bits(b_))  # bit patterns: the sentinel fill is a NaN in fp32
    assert torch.equal(pool, pool0), "verify wrote the committed state"
    log(f"ragged verify worst err {worst:.2e}")
    assert worst <= TOL


def test_verify_ragged_clamps_bounds(gpu):
    """Window bounds outside [0, total_tok], a decreasing step and a window longer than max_tok read as
    include/kda.h states (clamped, empty, cut): the outputs follow those windows and rows outside them
    are not written."""
    seed, H, L, S, R, max_tok = 91, 2, 1, 6, 16, 8
    cu = np.array([-4, 5, 3, 19, 40], dtype=np.int32)  # windows [0,5), empty, [3,11) cut from 16 rows, [19,20)
    total = 20
    B = len(cu) - 1
    slot_idx = torch.tensor([4, 0, 2, 5], dtype=torch.int32)
    pool = sg.states(seed, S * L * H, DEV).view(S, L, H, 128, 128)
    pool0 = pool.clone()
    ring_start = torch.tensor([0, 3, 9, 15], dtype=torch.int32)
    ring = kda.Ring.empty(S, L, H, R, DEV)
    for t in (ring.k, ring.v, ring.gk, ring.beta):
        t.view(torch.int16 if t.element_size() == 2 else torch.int32).fill_(-7)
    ring0 = kda.Ring(ring.k.clone(), ring.v.clone(), ring.gk.clone(), ring.beta.clone())
    ins = sg.prefill_inputs(seed, total, H, DEV)
    o = torch.full((total, H, 128), -9.0, device=DEV)
    assert [w for w in ragged_windows(cu, total, max_tok)] == [(0, 5), (5, 0), (3, 8), (19, 1)]
    kda.kda_verify_ragged(*ins, torch.from_numpy(cu).to(DEV), pool, slot_idx.to(DEV), o, layer=0, max_tok=max_tok,
                          ring=ring, ring_start=ring_start.to(DEV))
    torch.cuda.synchronize()
    # windows 0 and 2 share rows 3 and 4, so o is checked per window from separate calls below
    worst = 0.0
    for keep in ([0, 1, 3], [2]):
        cu_k = cu.copy()
        o_k = torch.full((total, H, 128), -9.0, device=DEV)
        sl = slot_idx.clone()
        for b in range(B):
            if b not in keep:
                sl[b] = -1
        ring_k = kda.Ring(ring0.k.clone(), ring0.v.clone(), ring0.gk.clone(), ring0.beta.clone())
        kda.kda_verify_ragged(*ins, torch.from_numpy(cu_k).to(DEV), pool, sl.to(DEV), o_k, layer=0, max_tok=max_tok,
                              ring=ring_k, ring_start=ring_start.to(DEV))
        torch.cuda.synchronize()
        worst = max(worst, check_ragged(0 + seed, 0, cu, total, max_tok, H, sl, pool0, o_k, ring_k, ring0, ring_start,
                                        R, 1.0))
    assert torch.equal(pool, pool0)
    assert np.all(np_(o)[11:19] == -9.0) and np.all(np_(o)[19] != -9.0)
    log(f"ragged verify with clamped bounds: worst err {worst:.2e}")
    assert worst <= TOL


@pytest.mark.parametrize("T,accs", [(8, [1, 2, 3, 4, 5, 6, 7, 8]), (1, [1, 0, 1, 1, 0, 1, 1, 0])])
def test_fold_bitexact_every_length(gpu, T, accs):
    seed, H, L, R = 40 + T, 3, 3, 16
    B = S = len(accs)
    log(f"fold bit-exact T={T}")
    slot_idx, pool, ins, ring_start = make_verify_case(seed, B, T, H, L, S, R)
    acc = torch.tensor(accs, dtype=torch.int32, device=DEV)
    ring = kda.Ring.empty(S, L, H, R, DEV)
    commit = pool.clone()
    for l in range(L):
        q, k, v, gk, beta = ins[l]
        o = torch.empty((B * T, H, 128), device=DEV)
        kda.kda_verify(q, k, v, gk, beta, pool, slot_idx.to(DEV), o, layer=l, n_tok=T, ring=ring,
                       ring_start=ring_start.to(DEV), commit_len=acc, commit_pool=commit)
    folded = pool.clone()
    kda.kda_replay_fold(folded, slot_idx.to(DEV), ring, acc, ring_start=ring_start.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(folded, commit)
    # against the oracle on a few units
    worst = 0.0
    for b in range(min(B, 3)):
        s = int(slot_idx[b])
        for l in range(L):
            q, k, v, gk, beta = host_inputs(seed, B, T, H, l, b, 1)
            n = int(acc[b])
            S_ref = oracle.fold(n, k, v, gk, beta, np.array(np_(pool[s, l, 1]), dtype=np.float64))
            worst = max(worst, block_err(np_(folded[s, l, 1]), S_ref))
    assert worst <= TOL


def test_verify_fp32_single_head_64(gpu):
    """Single sequence, 1 head, T = 64, fp32 everything, zero initial state (token-by-token path)."""
    log("single head x 64 tokens: verify on fp32 inputs")
    T, H = 64, 1
    q, k, v, gk, beta = sg.prefill_inputs(0, T, H, DEV, qkv_dtype=torch.float32)
    pool = torch.zeros((1, 1, H, 128, 128), device=DEV)
    commit = torch.empty_like(pool)
    o = torch.empty((T, H, 128), device=DEV)
    kda.kda_verify(q, k, v, gk, beta, pool, torch.zeros(1, dtype=torch.int32, device=DEV), o, layer=0, n_tok=T,
                   commit_len=torch.tensor([T], dtype=torch.int32, device=DEV), commit_pool=commit)
    torch.cuda.synchronize()
    hq, hk, hv, hg, hb = synth.prefill_rows(0, H, 0, T, h=0, qkv_dtype=synth.F32)
    o_ref, S_ref, _, _ = oracle.recurrent(hq, hk, hv, hg, hb)
    e_o, e_s = block_err(np_(o[:, 0]), o_ref), block_err(np_(commit[0, 0, 0]), S_ref)
    log(f"single head fp32 verify: o {e_o:.2e} state {e_s:.2e}")
    assert e_o <= TOL and e_s <= TOL


# ---------------------------------------------------------------- chunked prefill
def run_prefill(plan, ins, state_in=None, snap_slots=0, scale=1.0, flags=0, state_out=None, order_ws=None):
    q, k, v, gk, beta = ins
    N, H = plan.n_seq, plan.n_heads
    o = torch.full((plan.total_tokens, H, 128), float("nan"), device=DEV)
    if state_out is None:
        state_out = torch.empty((N, H, 128, 128), device=DEV)
    snap = torch.full((N, snap_slots, H, 128, 128), -5.0, device=DEV) if snap_slots else None
    cnt = torch.full((N,), -1, dtype=torch.int32, device=DEV)
    ws = order_ws if order_ws is not None else torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8,
                                                           device=DEV)
    kda.kda_chunk_prefill(plan, q, k, v, gk, beta, state_out, o, ws, state_in=state_in, snap=snap,
                          snap_slots=snap_slots, snap_count=cnt, scale=scale, flags=flags)
    return o, state_out, snap, cnt


def check_prefill(seed, plan, lens, H, o, st, snap, cnt, S0=None, scale=1.0, snap_slots=0, units=None):
    cu = plan.cu_seqlens
    worst = {"o": 0.0, "state": 0.0, "snap": 0.0}
    units = units if units is not None else [(n, h) for n in range(len(lens)) for h in range(H)]
    o_np, st_np = np_(o), np_(st)
    snap_np = np_(snap) if snap is not None else None
    for n, h in units:
        L = int(lens[n])
        s0 = None if S0 is None else S0[n, h]
        o_ref, S_ref, snaps_ref, c = oracle_prefill_unit(seed, H, int(cu[n]), L, h, S0=s0, scale=scale,
                                                         snap_interval=plan.snap_interval if snap_slots else 0,
                                                         snap_slots=snap_slots)
        if L > 0:
            worst["o"] = max(worst["o"], block_err(o_np[cu[n]:cu[n + 1], h], o_ref))
        worst["state"] = max(worst["state"], block_err(st_np[n, h], S_ref))
        if snap_slots:
            assert int(cnt[n]) == c
            for m in range(1, c + 1)[-snap_slots:]:
                sl = (m - 1) % snap_slots
                # the slot holds the latest snapshot written to it
                worst["snap"] = max(worst["snap"], block_err(snap_np[n, sl, h], snaps_ref[sl]))
    return worst


def test_prefill_ragged_small(gpu):
    seed, H = 11, 3
    lens = np.array([1, 31, 33, 100, 0, 257, 64])
    cu = synth.cu_seqlens(lens)
    log(f"prefill ragged lens={lens.tolist()}")
    plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=64)
    ins = sg.prefill_inputs(seed, int(cu[-1]), H, DEV)
    S0 = sg.states(seed, len(lens) * H, DEV).view(len(lens), H, 128, 128)
    o, st, snap, cnt = run_prefill(plan, ins, state_in=S0, snap_slots=2, scale=0.75)
    torch.cuda.synchronize()
    S0n = np_(S0)
    w = check_prefill(seed, plan, lens, H, o, st, snap, cnt, S0=S0n, scale=0.75, snap_slots=2)
    log(f"prefill ragged worst {w}")
    assert max(w.values()) <= TOL
    # sequences of length 0 keep their state
    assert torch.equal(st[4], S0[4])
    assert not torch.isnan(o).any()


@pytest.mark.parametrize("v_blocks", [2, 0])
def test_prefill_value_blocks_bitwise(gpu, v_blocks):
    """Items split into two value blocks of 64 columns give the same bits as whole (sequence, head)
    chains (o, state_out, snapshots, counts), on the ragged case the oracle checks above, with a
    state_in, snapshots and a scale; an automatic plan (v_blocks = 0) too."""
    seed, H = 11, 3
    lens = np.array([1, 31, 33, 100, 0, 257, 64])
    cu = synth.cu_seqlens(lens)
    ins = sg.prefill_inputs(seed, int(cu[-1]), H, DEV)
    S0 = sg.states(seed, len(lens) * H, DEV).view(len(lens), H, 128, 128)
    whole = kda.kda_plan_create(cu, n_heads=H, snap_interval=64)
    split = kda.kda_plan_create(cu, n_heads=H, snap_interval=64, v_blocks=v_blocks)
    log(f"prefill value blocks: plan with {kda.kda_plan_v_blocks(split)} block(s), {kda.kda_plan_num_items(split)} items")
    a = run_prefill(whole, ins, state_in=S0, snap_slots=2, scale=0.75)
    b = run_prefill(split, ins, state_in=S0, snap_slots=2, scale=0.75)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    if v_blocks == 2:
        assert kda.kda_plan_v_blocks(split) == 2


def test_prefill_single_head_64_bf16(gpu):
    """The single-head 64-token fp32 case through the chunked path on bf16-rounded q/k/v (the same draws)."""
    lens = np.array([64])
    plan = kda.kda_plan_create(synth.cu_seqlens(lens), n_heads=1)
    ins = sg.prefill_inputs(0, 64, 1, DEV)
    o, st, _, cnt = run_prefill(plan, ins)
    torch.cuda.synchronize()
    w = check_prefill(0, plan, lens, 1, o, st, None, cnt)
    log(f"single head x 64 tokens, chunked: {w}")
    assert max(w.values()) <= TOL


def test_prefill_exactness_properties(gpu):
    """NULL state_in == zeros; in place; run-to-run and LPT/FIFO determinism; resident
    work list reuse; a snapshot restores a chunk-aligned continuation bit for bit."""
    seed, H = 12, 2
    lens = np.array([96, 160, 7, 128])
    cu = synth.cu_seqlens(lens)
    N = len(lens)
    ins = sg.prefill_inputs(seed, int(cu[-1]), H, DEV)
    plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=64)
    o1, st1, sn1, _ = run_prefill(plan, ins, snap_slots=2)
    zeros = torch.zeros((N, H, 128, 128), device=DEV)
    o2, st2, _, _ = run_prefill(plan, ins, state_in=zeros, snap_slots=2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st1, st2)
    # in place
    S0 = sg.states(seed, N * H, DEV).view(N, H, 128, 128)
    o3, st3, _, _ = run_prefill(plan, ins, state_in=S0.clone(), snap_slots=2)
    inplace = S0.clone()
    o4, st4, _, _ = run_prefill(plan, ins, state_in=inplace, state_out=inplace, snap_slots=2)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(st3, inplace)
    # FIFO order and a resident work list give the same bits
    fifo = kda.kda_plan_create(cu, n_heads=H, snap_interval=64, order=kda.KDA_PLAN_FIFO)
    o5, st5, _, _ = run_prefill(fifo, ins, snap_slots=2)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    kda.kda_plan_upload(plan, ws)
    for _ in range(3):
        o6, st6, _, _ = run_prefill(plan, ins, snap_slots=2, flags=kda.KDA_PREFILL_PLAN_RESIDENT, order_ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(o6, o1) and torch.equal(st6, st1)
    assert torch.equal(o5, o1) and torch.equal(st5, st1)
    # restore: sequence 1 (160 tokens) from its snapshot at 128 continues identically
    sub_cu = np.array([0, 32], dtype=np.int32)
    sub = kda.kda_plan_create(sub_cu, n_heads=H)
    t0 = int(cu[1]) + 128
    sub_ins = tuple(x[t0:t0 + 32].contiguous() for x in ins)
    restored = sn1[1, 1].unsqueeze(0).contiguous()  # 128 = 2 * 64 -> slot (2 - 1) % 2 = 1
    o7, st7, _, _ = run_prefill(sub, sub_ins, state_in=restored)
    torch.cuda.synchronize()
    assert torch.equal(st7[0], st1[1]), "restored snapshot did not continue bit for bit"
    assert torch.equal(o7, o1[t0:t0 + 32])


# ---------------------------------------------------------------- output gated RMSNorm
TOL_NORM = 8e-3  # the pages' tolerance for the fast-math output norm (bf16 y, hardware exp/rcp/rsqrt)


def bf16_dev(bits_u16):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).view(torch.bfloat16).to(DEV)


def row_errs(y_bits, ref):
    """Per row of 128: max |y - ref| / max |ref| (rows of ref that are exactly zero must come out zero)."""
    y = (y_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(-1, 128)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, 128)
    den = np.max(np.abs(ref), axis=1)
    err = np.max(np.abs(y - ref), axis=1)
    assert np.all(err[den == 0] == 0)
    return err[den > 0] / den[den > 0]


def test_gated_rmsnorm_standalone(gpu):
    """kda_gated_rmsnorm against the oracle: 37 rows (a partial block), magnitudes from 1e-3 to 1e3, a zero
    row (eps > 0 sends it to zero), saturated gates, eps = 0 on the nonzero rows."""
    rng = np.random.default_rng(21)
    rows = 37
    o = (rng.standard_normal((rows, 128)) * rng.uniform(1e-3, 1e3, (rows, 1))).astype(np.float32)
    o[5] = 0.0
    gx = rng.standard_normal((rows, 128)) * 2.0
    gx[7], gx[8] = 30.0, -30.0
    gx[9, :64] = 40.0
    g_bits = synth.round_bf16(gx)
    w = synth.norm_weight(3)
    od, gd, wd = torch.from_numpy(o).to(DEV), bf16_dev(g_bits), torch.from_numpy(w).to(DEV)
    log("gated rmsnorm: standalone")
    for eps, sel in ((1e-6, np.arange(rows)), (0.0, np.delete(np.arange(rows), 5))):
        y = torch.empty((rows, 128), dtype=torch.bfloat16, device=DEV)
        kda.kda_gated_rmsnorm(od[sel].contiguous(), gd[sel].contiguous(), wd, eps, y[: len(sel)])
        torch.cuda.synchronize()
        ref = oracle.gated_rmsnorm(o[sel], g_bits[sel], w, eps)
        errs = row_errs(bits(y[: len(sel)]).view(np.uint16), ref)
        log(f"gated rmsnorm eps={eps}: worst row err {errs.max():.2e}")
        assert errs.max() <= TOL_NORM


def test_prefill_gated(gpu):
    """kda_chunk_prefill_gated on a ragged batch (empty, 1-token and partial-chunk sequences, state_in,
    snapshots): y bit-identical to kda_gated_rmsnorm applied to kda_chunk_prefill's o, the states and
    snapshots bit-identical to kda_chunk_prefill's, and y against the oracle (fp64 prefill, then the norm)
    on every (sequence, head); a two-value-block plan is refused."""
    seed, H, eps = 29, 3, 1e-6
    lens = [0, 1, 31, 33, 64, 100, 257]
    cu = synth.cu_seqlens(lens)
    T, N = int(cu[-1]), len(lens)
    plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=64)
    ins = sg.prefill_inputs(seed, T, H, DEV)
    gate = sg.gate(seed, T, H, DEV)
    w = synth.norm_weight(seed)
    wd = torch.from_numpy(w).to(DEV)
    S0 = sg.states(seed, N * H, DEV).view(N, H, 128, 128)
    log("gated prefill: plain prefill + standalone norm")
    o, st, snap, cnt = run_prefill(plan, ins, state_in=S0, snap_slots=2, scale=0.8)
    y_ref = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_gated_rmsnorm(o, gate, wd, eps, y_ref)
    log("gated prefill: fused")
    y = torch.full((T, H, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    st2 = torch.empty_like(st)
    snap2 = torch.full_like(snap, -5.0)
    cnt2 = torch.full_like(cnt, -1)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    kda.kda_chunk_prefill_gated(plan, *ins, gate, wd, eps, st2, y, ws, state_in=S0, snap=snap2, snap_slots=2,
                                snap_count=cnt2, scale=0.8)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y_ref)), "fused norm differs from prefill + kda_gated_rmsnorm"
    assert torch.equal(st2, st) and torch.equal(snap2, snap) and torch.equal(cnt2, cnt)
    yb = bits(y).view(np.uint16)
    worst = 0.0
    for n in range(N):
        t0, L = int(cu[n]), lens[n]
        if L == 0:
            continue
        for h in range(H):
            o_ref, _, _, _ = oracle_prefill_unit(seed, H, t0, L, h, S0=np_(S0[n, h]), scale=0.8)
            ref = oracle.gated_rmsnorm(o_ref, synth.gate_rows(seed, H, t0, L, h=h), w, eps)
            worst = max(worst, float(row_errs(yb[t0:t0 + L, h], ref).max()))
    log(f"gated prefill: worst row err {worst:.2e}")
    assert worst <= TOL_NORM
    split = kda.kda_plan_create(cu, n_heads=H, v_blocks=2)
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_prefill_gated(split, *ins, gate, wd, eps, st2, y, torch.empty(
            kda.kda_plan_workspace_bytes(split), dtype=torch.uint8, device=DEV))
    assert e.value.status == kda.KDA_ERR_UNSUPPORTED


# ---------------------------------------------------------------- the KDA prologue
def _prologue_inputs(rng, T, N, H, W):
    xs = [synth.round_bf16(rng.standard_normal((T, H, 128))) for _ in range(3)]
    conv_w = (0.5 * rng.standard_normal((3, H * 128, W))).astype(np.float32)
    st = synth.round_bf16(rng.standard_normal((N, 3, max(W - 1, 0), H * 128)))
    b = rng.standard_normal((T, H)).astype(np.float32)
    g = (2.0 * rng.standard_normal((T, H, 128))).astype(np.float32)
    return xs, conv_w, st, b, g


def _run_prologue(cu, xs, conv_w, st, b, g, eps, with_state=True):
    T, H = xs[0].shape[0], xs[0].shape[1]
    N, W = len(cu) - 1, conv_w.shape[2]
    dev = [bf16_dev(x) for x in xs]
    outs = [torch.full((T, H, 128), 3.0, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    beta = torch.full((T, H), -1.0, device=DEV)
    gk = torch.full((T, H, 128), 1.0, device=DEV)
    sin = bf16_dev(st) if with_state else None
    sout = torch.full((N, 3, W - 1, H * 128), 5.0, dtype=torch.bfloat16, device=DEV)
    kda.kda_prologue(torch.from_numpy(np.asarray(cu, dtype=np.int32)).to(DEV), *dev,
                     torch.from_numpy(conv_w).to(DEV), torch.from_numpy(b).to(DEV), torch.from_numpy(g).to(DEV),
                     *outs, beta, gk, conv_state_in=sin, conv_state_out=sout, eps=eps)
    torch.cuda.synchronize()
    return [bits(o).view(np.uint16) for o in outs], np_(beta), np_(gk), bits(sout).view(np.uint16)


@pytest.mark.parametrize("W", [4, 1, 2, 8])
def test_prologue(gpu, W):
    """kda_prologue on a ragged batch (lengths 0, 1, 2, 5, 40, 100 around the conv width) against the
    oracle per sequence: q, k, v per row at bf16 accuracy, beta and gk elementwise, the carried state bit
    for bit; without an incoming state it equals a zero state; a batch split in two calls, the first
    call's state feeding the second, gives the same bits as one call."""
    rng = np.random.default_rng(40 + W)
    H, eps = 3, 1e-6
    lens = [0, 1, 2, 5, 40, 100]
    cu = synth.cu_seqlens(lens)
    T, N = int(cu[-1]), len(lens)
    xs, conv_w, st, b, g = _prologue_inputs(rng, T, N, H, W)
    log(f"prologue W={W}")
    (q, k, v), beta, gk, sout = _run_prologue(cu, xs, conv_w, st, b, g, eps)
    worst = {"qkv": 0.0, "beta": 0.0, "gk": 0.0}
    for n in range(N):
        s0, L = int(cu[n]), lens[n]
        st_n = (st[n].astype(np.uint32) << 16).view(np.float32)  # the bf16 state rows, widened exactly
        ref = oracle.prologue(*(x[s0:s0 + L] for x in xs), conv_w, st_n, b[s0:s0 + L], g[s0:s0 + L], eps)
        for got, r in zip((q, k, v), ref[:3]):
            if L:
                worst["qkv"] = max(worst["qkv"], float(row_errs(got[s0:s0 + L], r).max()))
        if L:
            worst["beta"] = max(worst["beta"], float(np.max(np.abs(beta[s0:s0 + L] - ref[3]) / np.abs(ref[3]))))
            worst["gk"] = max(worst["gk"], float(np.max(np.abs(gk[s0:s0 + L] - ref[4]) / np.abs(ref[4]))))
        if W > 1:
            assert np.array_equal((sout[n].astype(np.uint32) << 16).view(np.float32), ref[5].astype(np.float32))
    log(f"prologue W={W}: worst {worst}")
    assert worst["qkv"] <= 5e-3 and worst["beta"] <= 1e-5 and worst["gk"] <= 1e-5
    # no incoming state = a zero state
    zero = np.zeros_like(st)
    a = _run_prologue(cu, xs, conv_w, st, b, g, eps, with_state=False)
    z = _run_prologue(cu, xs, conv_w, zero, b, g, eps)
    for x_, y_ in zip(a[0] + [a[3]], z[0] + [z[3]]):
        assert np.array_equal(x_, y_)
    # the batch in two calls with the state carried: sequence n's tokens split at m_n
    if W > 1:
        cut = [min(L, 3) for L in lens]
        first = [[x[int(cu[n]):int(cu[n]) + cut[n]] for n in range(N)] for x in xs]
        second = [[x[int(cu[n]) + cut[n]:int(cu[n + 1])] for n in range(N)] for x in xs]
        pick = lambda arr, parts: np.concatenate([arr[int(cu[n]) + lo:int(cu[n]) + hi] for n, (lo, hi) in enumerate(parts)])
        p1 = [(0, cut[n]) for n in range(N)]
        p2 = [(cut[n], lens[n]) for n in range(N)]
        c1, c2 = synth.cu_seqlens([c for c in cut]), synth.cu_seqlens([L - c for L, c in zip(lens, cut)])
        r1 = _run_prologue(c1, [np.concatenate(f) for f in first], conv_w, st, pick(b, p1), pick(g, p1), eps)
        r2 = _run_prologue(c2, [np.concatenate(f) for f in second], conv_w, r1[3], pick(b, p2), pick(g, p2), eps)
        for i in range(3):
            joined = np.concatenate([np.concatenate([r1[0][i][int(c1[n]):int(c1[n + 1])], r2[0][i][int(c2[n]):int(c2[n + 1])]])
                                     for n in range(N)])
            assert np.array_equal(joined, (q, k, v)[i])
        assert np.array_equal(r2[3], sout)


# ---------------------------------------------------------------- prefix-cache state moves
def test_state_move_bit_copy(gpu):
    """kda_state_move copies whole slots bit for bit (NaN and denormal patterns included); moves with a
    slot out of range or src == dst are skipped; every slot no move writes keeps its bits. Three slot
    sizes cover the unrolled body and the tail of the copy loop."""
    rng = np.random.default_rng(77)
    for S, per_slot in ((12, 2 * 3 * 128 * 128), (9, 4), (7, 4 * 1000 + 12)):
        bits0 = rng.integers(-2**31, 2**31, size=(S, per_slot), dtype=np.int64).astype(np.int32)
        pool = torch.from_numpy(bits0.copy()).to(DEV).view(torch.float32)
        dsts = rng.permutation(S)[:S // 2]
        srcs = [s for s in rng.permutation(S) if s not in set(dsts)][:len(dsts)]
        moves = [(int(a), int(b)) for a, b in zip(srcs, dsts)] + [(-1, 0), (0, S), (S + 3, 1), (2, 2), (1, -7)]
        log(f"state move: {S} slots x {per_slot} floats, {len(moves)} moves")
        kda.kda_state_move(pool, torch.tensor(moves, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        want = bits0.copy()
        for a, b in zip(srcs, dsts):
            want[b] = bits0[a]
        assert np.array_equal(pool.view(torch.int32).cpu().numpy(), want)


def test_prefix_cache_flow(gpu):
    """The three state moves around real prefills, one layer, H = 4. Request A prefills 700 tokens in
    checkpoint-aligned chunks (256, 256, 188), its working slot updated in place; after each chunk a
    snapshot, and the 256- and 512-token checkpoints donated to the tree. Request B shares A's first 512
    tokens: it restores the 512 checkpoint by copy-on-write and prefills its own 300 further tokens.
    Checks: each donated checkpoint equals a one-call prefill of that prefix bit for bit and is unchanged
    after B ran; B's outputs and final state equal a one-call prefill of its whole 812-token sequence bit
    for bit; and against the oracle on two heads (2e-3)."""
    H, seed_a, seed_b = 4, 31, 32
    pool_slots = kda.SlotPool(6)
    pool = torch.full((6, 1, H, 128, 128), float("nan"), device=DEV)

    def prefill(ins, L, state_in, state_out):
        plan = kda.kda_plan_create([0, L], n_heads=H)
        ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
        o = torch.empty((L, H, 128), device=DEV)
        kda.kda_chunk_prefill(plan, *ins, state_out, o, ws, state_in=state_in)
        return o

    def move(mv):
        kda.kda_state_move(pool.view(6, -1), torch.tensor([mv], dtype=torch.int32, device=DEV))

    A = sg.prefill_inputs(seed_a, 700, H, DEV)
    B_tail = sg.prefill_inputs(seed_b, 300, H, DEV)
    tree = {}
    ra, _ = pool_slots.open()
    w = ra.working
    pos = 0
    for L in kda.kda_chunk_split(0, 700, 300):
        log(f"prefix flow: A chunk [{pos}, {pos + L})")
        ins = [t[pos:pos + L] for t in A]
        prefill(ins, L, pool[w] if pos else None, pool[w])
        move(pool_slots.snapshot(ra))
        pos += L
        if pos % 256 == 0:
            tree[pos] = pool_slots.donate(ra)
    assert sorted(tree) == [256, 512]
    pool_slots.close(ra)
    torch.cuda.synchronize()
    ckpt = {p: pool[s].clone() for p, s in tree.items()}
    for p in (256, 512):
        ref = torch.empty((1, H, 128, 128), device=DEV)
        prefill([t[:p] for t in A], p, None, ref)
        torch.cuda.synchronize()
        assert torch.equal(ckpt[p].view(torch.int32), ref.view(torch.int32)), f"checkpoint {p} differs"

    rb, mv = pool_slots.open(tree[512])
    assert mv == [(tree[512], rb.working)]
    move(mv[0])
    log("prefix flow: B restores 512 and prefills 300")
    assert kda.kda_chunk_split(512, 300, 300) == [300]
    o_b = prefill(B_tail, 300, pool[rb.working], pool[rb.working])
    full = [torch.cat([a[:512], b]) for a, b in zip(A, B_tail)]
    st_full = torch.empty((1, H, 128, 128), device=DEV)
    o_full = prefill(full, 812, None, st_full)
    torch.cuda.synchronize()
    assert torch.equal(pool[tree[512]].view(torch.int32), ckpt[512].view(torch.int32)), "the tree's checkpoint changed"
    assert torch.equal(o_b.view(torch.int32), o_full[512:].view(torch.int32))
    assert torch.equal(pool[rb.working].view(torch.int32), st_full.view(torch.int32))
    for h in (0, 3):
        _, S512, _, _ = oracle_prefill_unit(seed_a, H, 0, 512, h)
        o_ref, S_end, _, _ = oracle_prefill_unit(seed_b, H, 0, 300, h, S0=S512)
        assert block_err(np_(o_b[:, h]), o_ref) <= TOL
        assert block_err(np_(pool[rb.working, 0, h]), S_end) <= TOL
    pool_slots.close(rb)


def test_prologue_empty_batch(gpu):
    """A batch whose sequences are all empty: no token outputs, and the carried state comes out equal to
    the state that went in, bit for bit (W = 4 and W = 8)."""
    rng = np.random.default_rng(9)
    for W in (4, 8):
        N, H = 3, 2
        st = synth.round_bf16(rng.standard_normal((N, 3, W - 1, H * 128)))
        conv_w = torch.zeros((3, H * 128, W), device=DEV)
        sout = torch.full((N, 3, W - 1, H * 128), 7.0, dtype=torch.bfloat16, device=DEV)
        e = torch.empty((0, H, 128), dtype=torch.bfloat16, device=DEV)
        kda.kda_prologue(torch.zeros(N + 1, dtype=torch.int32, device=DEV), e, e, e, conv_w,
                         torch.empty((0, H), device=DEV), torch.empty((0, H, 128), device=DEV),
                         torch.empty_like(e), torch.empty_like(e), torch.empty_like(e), torch.empty((0, H), device=DEV),
                         torch.empty((0, H, 128), device=DEV), conv_state_in=bf16_dev(st), conv_state_out=sout)
        torch.cuda.synchronize()
        assert np.array_equal(bits(sout).view(np.uint16), st)


def test_decode_graph_replay(gpu):
    """Single-token decode (kda_verify with n_tok = 1 and the commit written in place) captured as one HIP
    graph of 16 steps: three replays, each from the same starting state restored by eager work, with
    another eager decode run and synchronizations between them; every replay's outputs and final state
    equal the eager run's bit for bit."""
    H, steps, seed = 8, 16, 5
    tids = (synth.T_DEC_Q, synth.T_DEC_K, synth.T_DEC_V, synth.T_DEC_GK, synth.T_DEC_BETA)
    dq, dk, dv, dg, db = sg.prefill_inputs(seed, steps, H, DEV, tids=tids)
    start = sg.states(seed, H, DEV).view(1, 1, H, 128, 128)
    pool = start.clone()
    slot = torch.zeros(1, dtype=torch.int32, device=DEV)
    one = torch.ones(1, dtype=torch.int32, device=DEV)
    out = torch.empty((steps, H, 128), device=DEV)

    def decode(p, o):
        for t in range(steps):
            kda.kda_verify(dq[t:t + 1], dk[t:t + 1], dv[t:t + 1], dg[t:t + 1], db[t:t + 1], p, slot, o[t:t + 1],
                           layer=0, n_tok=1, commit_len=one, commit_pool=p)

    decode(pool, out)
    torch.cuda.synchronize()
    ref_o, ref_s = out.clone(), pool.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        decode(pool, out)
    other_pool, other_out = start.clone(), torch.empty_like(out)
    for r in range(3):
        log(f"decode graph: replay {r}")
        pool.copy_(start)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref_o.view(torch.int32)), f"replay {r}: outputs differ"
        assert torch.equal(pool.view(torch.int32), ref_s.view(torch.int32)), f"replay {r}: state differs"
        other_pool.copy_(start)
        decode(other_pool, other_out)   # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(other_out.view(torch.int32), ref_o.view(torch.int32))


def test_graph_replay_prefill_and_verify(gpu):
    """A ragged prefill (resident plan, state_in, snapshots) and two layers of speculative verify (the
    chunked path, ring written) each captured once as a HIP graph and replayed three times, with every
    output cleared by eager work and the same call run eagerly between replays: each replay equals the
    eager result bit for bit (outputs, states, snapshots, counts, ring)."""
    seed, H = 12, 3
    lens = [1, 31, 33, 100, 0, 257, 64]
    cu = synth.cu_seqlens(lens)
    T, N = int(cu[-1]), len(lens)
    plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=64)
    ins = sg.prefill_inputs(seed, T, H, DEV)
    S0 = sg.states(seed, N * H, DEV).view(N, H, 128, 128)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    kda.kda_plan_upload(plan, ws)
    o = torch.empty((T, H, 128), device=DEV)
    st = torch.empty((N, H, 128, 128), device=DEV)
    snap = torch.empty((N, 2, H, 128, 128), device=DEV)
    cnt = torch.empty((N,), dtype=torch.int32, device=DEV)
    pf_bufs = (o, st, snap, cnt)

    def prefill():
        kda.kda_chunk_prefill(plan, *ins, st, o, ws, state_in=S0, snap=snap, snap_slots=2, snap_count=cnt,
                              flags=kda.KDA_PREFILL_PLAN_RESIDENT)

    B, Tv, Hv, L, S, R = 5, 8, 4, 2, 8, 16
    slot_idx, pool, vins, ring_start = make_verify_case(seed, B, Tv, Hv, L, S, R)
    slot_idx, ring_start = slot_idx.to(DEV), ring_start.to(DEV)
    ring = kda.Ring.empty(S, L, Hv, R, DEV)
    vo = torch.empty((L, B * Tv, Hv, 128), device=DEV)
    vf_bufs = (vo, ring.k, ring.v, ring.gk, ring.beta)

    def verify():
        for l in range(L):
            kda.kda_verify(*vins[l], pool, slot_idx, vo[l], layer=l, n_tok=Tv, ring=ring, ring_start=ring_start)

    def clear(bufs):
        for t in bufs:
            t.fill_(-3) if t.dtype in (torch.int32, torch.int16) else t.fill_(float("nan"))

    def snapshot(bufs):
        return [t.view(torch.int16 if t.element_size() == 2 else torch.int32).clone() for t in bufs]

    for name, fn, bufs in (("prefill", prefill, pf_bufs), ("verify", verify, vf_bufs)):
        log(f"graph replay: {name}")
        if name == "verify":
            ring.k.zero_(); ring.v.zero_(); ring.gk.zero_(); ring.beta.zero_()
        outs = bufs if name == "prefill" else bufs[:1]  # cleared before each call (ring slots not written stay 0)
        clear(outs)
        fn()
        torch.cuda.synchronize()
        ref = snapshot(bufs)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for r in range(3):
            clear(outs)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for a, b in zip(snapshot(bufs), ref):
                assert torch.equal(a, b), f"{name}: replay {r} differs from the eager call"
            clear(outs)
            fn()  # the same call eagerly between replays
            torch.cuda.synchronize()
            for a, b in zip(snapshot(bufs), ref):
                assert torch.equal(a, b), f"{name}: eager call after replay {r} differs"


def test_plan_destroy_inside_capture(gpu):
    """Destroying plans while a graph is being captured (explicitly, and by the garbage collector
    finalizing a plan held in a reference cycle) leaves the capture valid: kda_plan_destroy makes no HIP
    call. The captured prefill, replayed, equals the eager call bit for bit; a later kda_host_release
    gives the queued pinned buffers back."""
    import gc
    lens = [33, 70]
    cu = synth.cu_seqlens(lens)
    T, N, H = int(cu[-1]), len(lens), 2
    plan = kda.kda_plan_create(cu, n_heads=H)
    ins = sg.prefill_inputs(13, T, H, DEV)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    kda.kda_plan_upload(plan, ws)
    o = torch.empty((T, H, 128), device=DEV)
    st = torch.empty((N, H, 128, 128), device=DEV)

    def prefill():
        kda.kda_chunk_prefill(plan, *ins, st, o, ws, flags=kda.KDA_PREFILL_PLAN_RESIDENT)

    prefill()
    torch.cuda.synchronize()
    ref = (o.clone(), st.clone())
    doomed = [kda.kda_plan_create(cu, n_heads=H) for _ in range(3)]
    cyc = {"plan": doomed[2]}
    cyc["self"] = cyc  # only the cyclic collector frees this one
    del doomed[2]
    log("plan destroy inside capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prefill()
        doomed[0].close()
        del doomed[1]
        del cyc
        gc.collect()
    for r in range(2):
        o.fill_(float("nan"))
        st.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int32), ref[0].view(torch.int32)), f"replay {r}: o"
        assert torch.equal(st.view(torch.int32), ref[1].view(torch.int32)), f"replay {r}: state"
    kda.kda_host_release()


def test_state_move_many_moves(gpu):
    """More moves than one grid dimension holds (70,000 > 65,535): the kernel strides over the moves.
    Slots of 4 floats; every even slot is copied to the next odd one, bit for bit."""
    n = 70000
    S = 2 * n
    rng = np.random.default_rng(3)
    bits0 = rng.integers(-2**31, 2**31, size=(S, 4), dtype=np.int64).astype(np.int32)
    pool = torch.from_numpy(bits0.copy()).to(DEV).view(torch.float32)
    moves = np.stack([np.arange(0, S, 2), np.arange(1, S, 2)], axis=1).astype(np.int32)
    kda.kda_state_move(pool, torch.from_numpy(moves).to(DEV))
    torch.cuda.synchronize()
    want = bits0.copy()
    want[1::2] = bits0[0::2]
    assert np.array_equal(pool.view(torch.int32).cpu().numpy(), want)


def test_prologue_clamps_bounds(gpu):
    """cu_seqlens out of range, decreasing or negative (a caller's bug): the kernels read every bound
    clamped into [0, T], so the call completes, every output is finite, and the first sequence, whose
    bounds are valid, matches a call with well-formed bounds bit for bit."""
    rng = np.random.default_rng(21)
    H, W, T = 2, 4, 64
    xs, conv_w, _, b, g = _prologue_inputs(rng, T, 4, H, W)
    st = synth.round_bf16(rng.standard_normal((4, 3, W - 1, H * 128)))
    bad = [0, 20, 10, 100000, T]           # sequence 1 decreasing, 2 past the end
    good = [0, 20, 40, 50, T]
    outs = {}
    for name, cu in (("bad", bad), ("good", good)):
        log(f"prologue clamps: {name} bounds {cu}")
        outs[name] = _run_prologue(cu, xs, conv_w, st, b, g, 1e-6)
    (q, k, v), beta, gk, sout = outs["bad"]
    for arr in (q, k, v):
        assert np.all(np.isfinite((arr.astype(np.uint32) << 16).view(np.float32)))
    assert np.all(np.isfinite(beta)) and np.all(np.isfinite(gk))
    assert np.all(np.isfinite((sout.astype(np.uint32) << 16).view(np.float32)))
    (qg, kg, vg), _, _, _ = outs["good"]
    for x_, y_ in ((q, qg), (k, kg), (v, vg)):
        assert np.array_equal(x_[:20], y_[:20])


@pytest.mark.parametrize("W", [4, 1, 2, 8])
def test_decode_fused(gpu, W):
    """kda_decode (prologue + step with in-place commit + gated RMSNorm in one launch) against the three
    launches it replaces: y, o, the committed pool and the conv state bit for bit; a request with no
    slot is skipped whole. End to end against the oracle (prologue, q/k/v rounded to bf16 as the
    recurrence takes them, the recurrence, the norm): state 2e-3, y 8e-3 per row."""
    rng = np.random.default_rng(60 + W)
    B, H, Lyr, S, layer, eps = 3, 4, 2, 6, 1, 1e-6
    xs = [synth.round_bf16(rng.standard_normal((B, H, 128))) for _ in range(3)]
    conv_w = (0.5 * rng.standard_normal((3, H * 128, W))).astype(np.float32)
    cs0 = synth.round_bf16(rng.standard_normal((B, 3, W - 1, H * 128)))
    b = rng.standard_normal((B, H)).astype(np.float32)
    g = (2.0 * rng.standard_normal((B, H, 128))).astype(np.float32)
    gate = synth.round_bf16(rng.standard_normal((B, H, 128)))
    nw = (1.0 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    slots = torch.tensor([4, -1, 1], dtype=torch.int32, device=DEV)
    pool0 = sg.states(60 + W, S * Lyr * H, DEV).view(S, Lyr, H, 128, 128)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    xd = [bf16_dev(x) for x in xs]
    wd, bd, gd, gated, nwd = dev(conv_w), dev(b), dev(g), bf16_dev(gate), dev(nw)
    log(f"decode fused W={W}")
    # fused
    pool_f, cs_f = pool0.clone(), bf16_dev(cs0)
    y_f = torch.full((B, H, 128), 9.0, dtype=torch.bfloat16, device=DEV)
    o_f = torch.full((B, H, 128), 9.0, device=DEV)
    kda.kda_decode(*xd, wd, cs_f if W > 1 else None, bd, gd, pool_f, slots, gated, nwd, y_f, layer=layer, o=o_f,
                   qk_eps=eps, norm_eps=eps)
    # the chain it replaces
    pool_c = pool0.clone()
    q, k, v = (torch.empty((B, H, 128), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    beta, gk = torch.empty((B, H), device=DEV), torch.empty((B, H, 128), device=DEV)
    cs_out = torch.empty((B, 3, W - 1, H * 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_prologue(torch.arange(B + 1, dtype=torch.int32, device=DEV), *xd, wd, bd, gd, q, k, v, beta, gk,
                     conv_state_in=bf16_dev(cs0) if W > 1 else None, conv_state_out=cs_out if W > 1 else None, eps=eps)
    o_c = torch.full((B, H, 128), 9.0, device=DEV)
    one = torch.ones(B, dtype=torch.int32, device=DEV)
    kda.kda_verify(q, k, v, gk, beta, pool_c, slots, o_c, layer=layer, n_tok=1, commit_len=one, commit_pool=pool_c)
    y_c = torch.empty((B, H, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_gated_rmsnorm(o_c, gated, nwd, eps, y_c)
    torch.cuda.synchronize()
    ok = [0, 2]
    assert torch.equal(y_f[ok].view(torch.int16), y_c[ok].view(torch.int16))
    assert torch.equal(o_f[ok].view(torch.int32), o_c[ok].view(torch.int32))
    assert torch.equal(pool_f.view(torch.int32), pool_c.view(torch.int32))
    assert torch.all(y_f[1].float() == 9.0) and torch.all(o_f[1] == 9.0)
    if W > 1:
        csf = bits(cs_f).view(np.uint16)
        assert np.array_equal(csf[ok], bits(cs_out).view(np.uint16)[ok])
        assert np.array_equal(csf[1], cs0[1])
    # end to end against the oracle
    worst_s, worst_y = 0.0, 0.0
    yb = bits(y_f).view(np.uint16)
    for r, s in ((0, 4), (2, 1)):
        st = (cs0[r].astype(np.uint32) << 16).view(np.float32) if W > 1 else np.zeros((3, 0, H * 128))
        qo, ko, vo, bo, go, _ = oracle.prologue(*(x[r:r + 1] for x in xs), conv_w, st, b[r:r + 1], g[r:r + 1], eps)
        for h in range(H):
            qh, kh, vh = (synth.bf16_to_f64(synth.round_bf16(t[:, h])) for t in (qo, ko, vo))
            o_ref, S_ref, _, _ = oracle.recurrent(qh, kh, vh, go[:, h], bo[:, h], np_(pool0[s, layer, h]))
            y_ref = oracle.gated_rmsnorm(o_ref, synth.bf16_to_f64(gate[r:r + 1, h]), nw, eps)
            worst_s = max(worst_s, block_err(np_(pool_f[s, layer, h]), S_ref))
            yv = synth.bf16_to_f64(yb[r, h])
            worst_y = max(worst_y, float(np.max(np.abs(yv - y_ref[0])) / np.max(np.abs(y_ref[0]))))
    log(f"decode fused W={W}: worst state {worst_s:.2e}, y {worst_y:.2e}")
    assert worst_s <= TOL and worst_y <= 8e-3


def test_probes(gpu):
    """The measurement probes do the work they report: the copy reproduces its source bit for bit, the
    read's per-thread sums add up to the source's sum, and every thread of the MFMA loop ends with
    iters x 8 accumulators x the sum of its four entries of A B, where lane l holds A[l % 16][8 (l / 16) + i]
    = bf16(seed (l + i)) and B[8 (l / 16) + i][l % 16] = bf16(seed (l - i)) and gets D[4 (l / 16) + r][l % 16]."""
    n = 1 << 22
    src = torch.randn(n, device=DEV)
    dst = torch.empty_like(src)
    kda.kda_probe_copy(dst, src)
    sink = torch.zeros(2048 * 256, device=DEV)
    kda.kda_probe_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    total, mag = float(src.double().sum()), float(src.abs().double().sum())
    assert abs(float(sink.double().sum()) - total) <= 1e-5 * mag
    # MFMA loop
    iters, seed = 64, 1e-3  # a multiple of the probe's 32-round blocks (other counts round up)
    assert kda.kda_probe_mfma(33, sink, seed=seed) == kda.kda_probe_mfma(64, sink, seed=seed)
    sink.zero_()
    flop = kda.kda_probe_mfma(iters, sink, seed=seed)
    torch.cuda.synchronize()
    grid = flop // (4 * 8 * iters * 2 * 16 * 16 * 32)
    assert grid >= 1 and flop == grid * 4 * 8 * iters * 2 * 16 * 16 * 32
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    bf = lambda x: float(torch.tensor(np.float32(x)).to(torch.bfloat16).double())
    for l in range(64):
        g, lr = divmod(l, 16)
        for i in range(8):
            A[lr, 8 * g + i] = bf(np.float32(seed) * np.float32(l + i))
            B[8 * g + i, lr] = bf(np.float32(seed) * np.float32(l - i))
    Dm = A @ B
    per_lane = np.array([iters * 8 * sum(Dm[4 * (l // 16) + r, l % 16] for r in range(4)) for l in range(64)])
    got = np_(sink[: grid * 256]).reshape(grid * 4, 64).astype(np.float64)
    err = np.abs(got - per_lane[None, :]).max() / np.abs(per_lane).max()
    log(f"probes: mfma grid {grid}, worst relative error {err:.2e}")
    assert err <= 1e-5
