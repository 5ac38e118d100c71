"""Edge cases of the method on the chunked paths (the prefill and the served chunked verify), through
the C ABI, against the fp64 oracle on exactly the values the kernels consume:

  i1      beta = 0, gk = 0: the state is unchanged (bit for bit on the prefill) and o = scale S0^T q
  i5      beta = 1 and one-hot k (unit norm exactly): the delta rule writes v at key k, S_t^T k_t = v_t
  i8      gk = -inf: every token resets the state, S_t = beta_t k_t v_t^T
  bound   gk = -5 everywhere: 80 of decay over each 16-token half, the edge of the factor form
  past    gk = -7 everywhere: beyond it (the exact path)
  mixed   the workloads' gk with 2% of entries -inf and 5% at -30
  large   state_in ~ N(0, 300^2) and v ~ N(0, 30^2)

Inputs are drawn on the host (numpy, seeded) and rounded to the kernels' dtypes; q rows are unit
vectors, k rows unit vectors (one-hot in i5), beta = sigmoid(N(0,1)) unless the case fixes it.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.gpu as sg
import linear_attention_recurrence_amd as kda
from kda_ref import TOL, block_err, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CASES = ["i1", "i5", "i8", "bound", "past", "mixed", "large"]


def _unit_rows(rng, n):
    x = rng.standard_normal((n, 128))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def make_inputs(case, rng, rows):
    """q, k, v as bf16 bits [rows, 128]; gk, beta fp32; and the state scale for this case."""
    q = synth.round_bf16(_unit_rows(rng, rows))
    if case == "i5":
        kk = np.zeros((rows, 128))
        kk[np.arange(rows), rng.integers(0, 128, rows)] = 1.0
        k = synth.round_bf16(kk)
    else:
        k = synth.round_bf16(_unit_rows(rng, rows))
    v = synth.round_bf16(rng.standard_normal((rows, 128)) * (30.0 if case == "large" else 1.0))
    gk = -np.logaddexp(0.0, rng.standard_normal((rows, 128)))  # -softplus(N(0,1))
    if case == "i1":
        gk[:] = 0.0
    elif case == "i8":
        gk[:] = -np.inf
    elif case == "bound":
        gk[:] = -5.0
    elif case == "past":
        gk[:] = -7.0
    elif case == "mixed":
        u = rng.random((rows, 128))
        gk[u < 0.02] = -np.inf
        gk[(u >= 0.02) & (u < 0.07)] = -30.0
    gk = gk.astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal(rows)))).astype(np.float32)
    if case == "i1":
        beta[:] = 0.0
    elif case == "i5":
        beta[:] = 1.0
    sscale = 300.0 if case == "large" else 0.1
    return q, k, v, gk, beta, sscale


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


@pytest.mark.parametrize("v_blocks", [1, 2])
@pytest.mark.parametrize("case", CASES)
def test_prefill_edge(gpu, case, v_blocks):
    """kda_chunk_prefill on a ragged batch (lengths 1, 40, 100, 0, 65: several chunks, partial last
    chunks, an empty sequence) with state_in and snapshots every 32 tokens, against the oracle per
    (sequence, head): o, state, last snapshot; i1 also bit for bit (state_out == state_in)."""
    rng = np.random.default_rng(1000 + CASES.index(case))
    lens, H = [1, 40, 100, 0, 65], 2
    cu = synth.cu_seqlens(lens)
    T, N = int(cu[-1]), len(lens)
    q, k, v, gk, beta, sscale = make_inputs(case, rng, T * H)
    S0 = (rng.standard_normal((N, H, 128, 128)) * sscale).astype(np.float32)
    shp = (T, H, 128)
    ins = (bf16_dev(q.reshape(shp)), bf16_dev(k.reshape(shp)), bf16_dev(v.reshape(shp)), f32_dev(gk.reshape(shp)),
           f32_dev(beta.reshape(T, H)))
    plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=32, v_blocks=v_blocks)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    o = torch.full(shp, float("nan"), device=DEV)
    st = torch.full((N, H, 128, 128), float("nan"), device=DEV)
    snap = torch.full((N, 2, H, 128, 128), float("nan"), device=DEV)
    log(f"prefill edge case {case}, value blocks {v_blocks}")
    kda.kda_chunk_prefill(plan, *ins, st, o, ws, state_in=f32_dev(S0), snap=snap, snap_slots=2)
    torch.cuda.synchronize()
    o_np, st_np, sn_np = o.cpu().numpy(), st.cpu().numpy(), snap.cpu().numpy()
    assert np.all(np.isfinite(o_np)) and np.all(np.isfinite(st_np))
    if case == "i1":
        assert np.array_equal(st_np.view(np.int32), S0.view(np.int32)), "beta = 0, gk = 0 must leave the state unchanged"
    worst = {"o": 0.0, "state": 0.0, "snap": 0.0}
    q3, k3, v3, g3, b2 = q.reshape(shp), k.reshape(shp), v.reshape(shp), gk.reshape(shp), beta.reshape(T, H)
    for n in range(N):
        a, e = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            o_ref, S_ref, snaps, cnt = oracle.recurrent(q3[a:e, h], k3[a:e, h], v3[a:e, h], g3[a:e, h], b2[a:e, h],
                                                        S0[n, h], snap_interval=32, snap_slots=2)
            if e > a:
                worst["o"] = max(worst["o"], block_err(o_np[a:e, h], o_ref))
            worst["state"] = max(worst["state"], block_err(st_np[n, h], S_ref))
            if cnt:
                sl = (cnt - 1) % 2
                worst["snap"] = max(worst["snap"], block_err(sn_np[n, sl, h], snaps[sl]))
            if case == "i8" and e > a:  # closed form: the last token alone
                kl = synth.bf16_to_f64(k3[e - 1, h])
                vl = synth.bf16_to_f64(v3[e - 1, h])
                assert block_err(st_np[n, h], float(b2[e - 1, h]) * np.outer(kl, vl)) <= TOL
            if case == "i5" and e > a:  # the delta rule writes v at key k
                kl = synth.bf16_to_f64(k3[e - 1, h])
                vl = synth.bf16_to_f64(v3[e - 1, h])
                assert block_err(st_np[n, h].T.astype(np.float64) @ kl, vl) <= TOL
    log(f"prefill edge case {case}, value blocks {v_blocks}: worst {worst}")
    assert max(worst.values()) <= TOL, worst
    plan.close()


@pytest.mark.parametrize("v_blocks", [1, 2])
def test_prefill_rerun(gpu, v_blocks):
    """A batch where one sequence's chunks leave the factor form's range (the mixed case's gk) and the
    others' do not: the kernel computes the flagged items a second time, in the form with the exact
    path. With state_out == state_in (in place) that second pass must still read the initial state: o,
    the final states and the snapshots equal the out-of-place call's bit for bit, and every (sequence,
    head) agrees with the oracle. With one value block the fused gated call, which takes the same
    second pass, gives y equal to kda_gated_rmsnorm of the plain call's o and the same states."""
    rng = np.random.default_rng(4000 + v_blocks)
    lens, H, flagged = [70, 97, 33], 2, 1
    cu = synth.cu_seqlens(lens)
    T, N = int(cu[-1]), len(lens)
    q, k, v, gk, beta, _ = make_inputs("mixed", rng, T * H)
    shp = (T, H, 128)
    gk = gk.reshape(shp)
    plain = (-np.logaddexp(0.0, rng.standard_normal(shp))).astype(np.float32)
    for n in range(N):
        if n != flagged:
            gk[cu[n]:cu[n + 1]] = plain[cu[n]:cu[n + 1]]
    S0 = (rng.standard_normal((N, H, 128, 128)) * 0.1).astype(np.float32)
    ins = (bf16_dev(q.reshape(shp)), bf16_dev(k.reshape(shp)), bf16_dev(v.reshape(shp)), f32_dev(gk),
           f32_dev(beta.reshape(T, H)))
    plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=32, v_blocks=v_blocks)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)

    def call(state_in, state_out):
        o = torch.full(shp, float("nan"), device=DEV)
        snap = torch.full((N, 2, H, 128, 128), float("nan"), device=DEV)
        kda.kda_chunk_prefill(plan, *ins, state_out, o, ws, state_in=state_in, snap=snap, snap_slots=2)
        return o, snap

    log(f"prefill second pass, value blocks {v_blocks}: out of place, then in place")
    st_a = torch.full((N, H, 128, 128), float("nan"), device=DEV)
    o_a, sn_a = call(f32_dev(S0), st_a)
    inplace = f32_dev(S0)
    o_b, sn_b = call(inplace, inplace)
    torch.cuda.synchronize()
    o_np, st_np, sn_np = o_a.cpu().numpy(), st_a.cpu().numpy(), sn_a.cpu().numpy()
    assert np.all(np.isfinite(o_np)) and np.all(np.isfinite(st_np))
    bits = lambda t: t.view(torch.int32)  # noqa: E731 (unused snapshot slots stay NaN: compare bits)
    assert torch.equal(bits(o_a), bits(o_b)) and torch.equal(bits(st_a), bits(inplace)) \
        and torch.equal(bits(sn_a), bits(sn_b)), "the in-place call differs from the out-of-place one"
    worst = {"o": 0.0, "state": 0.0, "snap": 0.0}
    q3, k3, v3, b2 = q.reshape(shp), k.reshape(shp), v.reshape(shp), beta.reshape(T, H)
    for n in range(N):
        a, e = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            o_ref, S_ref, snaps, cnt = oracle.recurrent(q3[a:e, h], k3[a:e, h], v3[a:e, h], gk[a:e, h], b2[a:e, h],
                                                        S0[n, h], snap_interval=32, snap_slots=2)
            worst["o"] = max(worst["o"], block_err(o_np[a:e, h], o_ref))
            worst["state"] = max(worst["state"], block_err(st_np[n, h], S_ref))
            sl = (cnt - 1) % 2
            worst["snap"] = max(worst["snap"], block_err(sn_np[n, sl, h], snaps[sl]))
    log(f"prefill second pass, value blocks {v_blocks}: worst {worst}")
    assert max(worst.values()) <= TOL, worst
    if v_blocks == 1:
        gate = sg.gate(4000, T, H, DEV)
        wd = torch.from_numpy(synth.norm_weight(4000)).to(DEV)
        y_ref = torch.empty(shp, dtype=torch.bfloat16, device=DEV)
        kda.kda_gated_rmsnorm(o_a, gate, wd, 1e-6, y_ref)
        y = torch.full(shp, 7.0, dtype=torch.bfloat16, device=DEV)
        st_g = f32_dev(S0)
        sn_g = torch.full((N, 2, H, 128, 128), float("nan"), device=DEV)
        log("prefill second pass, gated, in place")
        kda.kda_chunk_prefill_gated(plan, *ins, gate, wd, 1e-6, st_g, y, ws, state_in=st_g, snap=sn_g, snap_slots=2)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), "fused norm differs from prefill + norm"
        assert torch.equal(bits(st_g), bits(st_a)) and torch.equal(bits(sn_g), bits(sn_a))
    plan.close()


@pytest.mark.parametrize("n_tok", [8, 16])
@pytest.mark.parametrize("case", CASES)
def test_verify_chunk_edge(gpu, case, n_tok):
    """kda_verify without a commit (the chunked matrix-core path the speculative step serves) with the
    ring: o against the oracle per (request, head), the ring entries equal to the inputs bit for bit
    (-inf included), the pool untouched; then kda_replay_fold of every recorded length equals the
    token-by-token kernel's commit bit for bit and the oracle's n steps."""
    rng = np.random.default_rng(2000 + 10 * n_tok + CASES.index(case))
    B, H, S, R = 5, 2, 7, 2 * n_tok
    rows = B * n_tok * H
    q, k, v, gk, beta, sscale = make_inputs(case, rng, rows)
    shp = (B * n_tok, H, 128)
    ins = (bf16_dev(q.reshape(shp)), bf16_dev(k.reshape(shp)), bf16_dev(v.reshape(shp)), f32_dev(gk.reshape(shp)),
           f32_dev(beta.reshape(B * n_tok, H)))
    pool0 = (rng.standard_normal((S, 1, H, 128, 128)) * sscale).astype(np.float32)
    pool = f32_dev(pool0)
    slots = np.array([3, 0, 6, 1, 4], dtype=np.int32)
    slot_idx = torch.from_numpy(slots).to(DEV)
    ring_start = torch.from_numpy(rng.integers(0, 3 * R, B).astype(np.int32)).to(DEV)
    ring = kda.Ring.empty(S, 1, H, R, DEV)
    o = torch.full(shp, float("nan"), device=DEV)
    log(f"verify edge case {case}, n_tok {n_tok}")
    kda.kda_verify(*ins, pool, slot_idx, o, layer=0, n_tok=n_tok, ring=ring, ring_start=ring_start)
    # the token-by-token verify with a commit of every length, for the fold's bit-exact reference
    acc = np.array([n_tok, 1, 0, n_tok // 2, 3], dtype=np.int32)
    commit = pool.clone()
    o2 = torch.empty_like(o)
    kda.kda_verify(*ins, pool, slot_idx, o2, layer=0, n_tok=n_tok, commit_len=torch.from_numpy(np.maximum(acc, 1)).to(DEV),
                   commit_pool=commit)
    folded = pool.clone()
    kda.kda_replay_fold(folded, slot_idx, ring, torch.from_numpy(acc).to(DEV), ring_start=ring_start)
    torch.cuda.synchronize()
    assert torch.equal(pool.view(torch.int32), f32_dev(pool0).view(torch.int32)), "verify wrote the committed pool"
    o_np = o.cpu().numpy()
    assert np.all(np.isfinite(o_np))
    rs = ring_start.cpu().numpy()
    rk, rv = ring.k.view(torch.int16).cpu().numpy(), ring.v.view(torch.int16).cpu().numpy()
    rg, rb = ring.gk.cpu().numpy(), ring.beta.cpu().numpy()
    q3, k3, v3, g3, b2 = q.reshape(shp), k.reshape(shp), v.reshape(shp), gk.reshape(shp), beta.reshape(B * n_tok, H)
    fol, com = folded.cpu().numpy(), commit.cpu().numpy()
    worst = 0.0
    for b in range(B):
        s = int(slots[b])
        r0, r1 = b * n_tok, (b + 1) * n_tok
        for h in range(H):
            o_ref, _, _ = oracle.verify(q3[r0:r1, h], k3[r0:r1, h], v3[r0:r1, h], g3[r0:r1, h], b2[r0:r1, h],
                                        pool0[s, 0, h])
            worst = max(worst, block_err(o_np[r0:r1, h], o_ref))
            for t in range(n_tok):
                pos = (int(rs[b]) + t) & (R - 1)
                assert np.array_equal(rk[s, 0, h, pos], k3[r0 + t, h].view(np.int16))
                assert np.array_equal(rv[s, 0, h, pos], v3[r0 + t, h].view(np.int16))
                assert np.array_equal(rg[s, 0, h, pos].view(np.int32), g3[r0 + t, h].view(np.int32))
                assert rb[s, 0, h, pos].view(np.int32) == b2[r0 + t, h].view(np.int32)
            n = int(acc[b])
            if n == 0:
                assert np.array_equal(fol[s, 0, h].view(np.int32), pool0[s, 0, h].view(np.int32))
            else:
                assert np.array_equal(fol[s, 0, h].view(np.int32), com[s, 0, h].view(np.int32)), \
                    f"fold of {n} steps differs from the commit (request {b}, head {h})"
                _, S_ref, _ = oracle.verify(q3[r0:r0 + n, h], k3[r0:r0 + n, h], v3[r0:r0 + n, h], g3[r0:r0 + n, h],
                                            b2[r0:r0 + n, h], pool0[s, 0, h], commit_len=n, record=False)
                worst = max(worst, block_err(fol[s, 0, h], S_ref))
    log(f"verify edge case {case}, n_tok {n_tok}: worst {worst:.2e}")
    assert worst <= TOL, worst


@pytest.mark.parametrize("case", ["i8", "past", "mixed"])
def test_fold_verify_edge(gpu, case):
    """kda_fold_verify (fold the previous window, then verify the next from the folded state) on decays
    beyond the factor form's range equals kda_replay_fold followed by kda_verify bit for bit."""
    rng = np.random.default_rng(3000 + CASES.index(case))
    B, H, S, T, R = 4, 2, 6, 8, 16
    rows = B * T * H
    shp = (B * T, H, 128)
    wins = []
    for _ in range(2):
        q, k, v, gk, beta, sscale = make_inputs(case, rng, rows)
        wins.append((bf16_dev(q.reshape(shp)), bf16_dev(k.reshape(shp)), bf16_dev(v.reshape(shp)),
                     f32_dev(gk.reshape(shp)), f32_dev(beta.reshape(B * T, H))))
    pool0 = f32_dev((rng.standard_normal((S, 1, H, 128, 128)) * 0.1).astype(np.float32))
    slot_idx = torch.tensor([5, 2, 0, 3], dtype=torch.int32, device=DEV)
    acc = torch.tensor([3, 8, 1, 5], dtype=torch.int32, device=DEV)
    start0 = torch.zeros(B, dtype=torch.int32, device=DEV)
    start1 = torch.full((B,), T, dtype=torch.int32, device=DEV)
    log(f"fold-verify edge case {case}")
    outs = []
    for fused in (False, True):
        pool = pool0.clone()
        ring = kda.Ring.empty(S, 1, H, R, DEV)
        for t in (ring.k, ring.v, ring.gk, ring.beta):
            t.zero_()  # rows of slots no request uses stay zero in both runs
        o0 = torch.empty(shp, device=DEV)
        kda.kda_verify(*wins[0], pool, slot_idx, o0, layer=0, n_tok=T, ring=ring, ring_start=start0)
        o1 = torch.full(shp, float("nan"), device=DEV)
        if fused:
            kda.kda_fold_verify(*wins[1], pool, slot_idx, o1, layer=0, n_tok=T, ring=ring, fold_len=acc,
                                fold_start=start0, ring_start=start1)
        else:
            kda.kda_replay_fold(pool, slot_idx, ring, acc, ring_start=start0)
            kda.kda_verify(*wins[1], pool, slot_idx, o1, layer=0, n_tok=T, ring=ring, ring_start=start1)
        torch.cuda.synchronize()
        outs.append([t.view(torch.int32).clone() for t in (pool, o1, ring.gk)])
    for a, b, name in zip(outs[0], outs[1], ("pool", "o", "ring gk")):
        assert torch.equal(a, b), f"{case}: {name} differs"
    assert torch.all(torch.isfinite(outs[1][1].view(torch.float32)))
