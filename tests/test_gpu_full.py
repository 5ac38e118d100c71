"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times, through the C ABI. The oracle covers every unit where it
finishes in seconds, a stated sample elsewhere (the whole longest and
shortest sequences plus random units; two full heads of the 1M-token run);
bit-exact properties are checked on every unit.

Workloads (synthetic, seeded, shapes from the pages; K = V = 128):
  prefill A: 4 x 2048 tokens, H = 64, state_in ~ N(0, 0.1^2)
  prefill B: 32 sequences, lengths log-uniform in [64, 24576], H = 96,
             snapshots every 2048 tokens into 2 ping-pong slots
  spec step: 256 requests x 69 layers x 8 heads, gamma + 1 = 8, ring 16,
             accepted lengths geometric (mean 2.7, clipped to [1, 8])
  long:      1 x 1,048,576 tokens, H = 96, snapshots every 4096 into 2
             slots, then 128 single-token decode steps
  prologue:  the 4 x 2048, H = 64 batch through kda_prologue, conv width 4
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.gpu as sg
import linear_attention_recurrence_amd as kda
from kda_ref import TOL, block_err, log, oracle_prefill_unit, threads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def np_(t):
    return t.detach().cpu().numpy()


def rows_err(x, ref, rows):
    """Worst normwise error over blocks of `rows` consecutive tokens (max |x - r| / max |r| within each
    block): a local error in a low-magnitude stretch cannot hide under the whole sequence's maximum."""
    n = (len(ref) // rows) * rows
    xb = np.asarray(x[:n], dtype=np.float64).reshape(-1, rows * ref.shape[1])
    rb = np.asarray(ref[:n], dtype=np.float64).reshape(-1, rows * ref.shape[1])
    den = np.maximum(np.max(np.abs(rb), axis=1), 1e-30)
    worst = float(np.max(np.max(np.abs(xb - rb), axis=1) / den)) if n else 0.0
    if n < len(ref):
        worst = max(worst, block_err(x[n:], ref[n:]))
    return worst


def prefill_launch(plan, ins, o, st, snap, cnt, snap_slots, state_in=None):
    """One prefill with a resident work list; returns its time in ms (HIP events)."""
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    kda.kda_plan_upload(plan, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    kda.kda_chunk_prefill(plan, *ins, st, o, ws, state_in=state_in, snap=snap, snap_slots=snap_slots,
                          snap_count=cnt, flags=kda.KDA_PREFILL_PLAN_RESIDENT)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def prefill_run(cfg, lens, H, state_in=None, snap_slots=0, order=kda.KDA_PLAN_LPT, v_blocks=1):
    c = synth.PREFILL_CONFIGS[cfg]
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=c["snap_interval"], order=order, v_blocks=v_blocks)
    ins = sg.prefill_inputs(c["seed"], T, H, DEV)
    N = len(lens)
    o = torch.empty((T, H, 128), device=DEV)
    st = torch.empty((N, H, 128, 128), device=DEV)
    snap = torch.full((N, snap_slots, H, 128, 128), -5.0, device=DEV) if snap_slots else None
    cnt = torch.full((N,), -1, dtype=torch.int32, device=DEV)
    ms = prefill_launch(plan, ins, o, st, snap, cnt, snap_slots, state_in=state_in)
    log(f"prefill {cfg}: {kda.kda_plan_num_items(plan)} items ({kda.kda_plan_v_blocks(plan)} value "
        f"block(s) each), {ms:.2f} ms")
    return plan, cu, ins, o, st, snap, cnt


def check_units(cfg, cu, H, units, o, st, snap=None, snap_slots=0, S0=None, interval=0):
    seed = synth.PREFILL_CONFIGS[cfg]["seed"]
    o_np = {}
    for n, h in units:  # device -> host slices first (one process, sequential)
        o_np[(n, h)] = np_(o[int(cu[n]):int(cu[n + 1]), h])
    st_np = np_(st)
    sn_np = np_(snap) if snap is not None else None

    def run(u):
        n, h = u
        L = int(cu[n + 1] - cu[n])
        s0 = None if S0 is None else S0[n, h]
        o_ref, S_ref, sn_ref, c = oracle_prefill_unit(seed, H, int(cu[n]), L, h, S0=s0, snap_interval=interval,
                                                      snap_slots=snap_slots)
        e = {"o": block_err(o_np[u], o_ref) if L else 0.0, "o_64": rows_err(o_np[u], o_ref, 64) if L else 0.0,
             "state": block_err(st_np[n, h], S_ref), "snap": 0.0, "count": c}
        for m in range(max(1, c - snap_slots + 1), c + 1):
            sl = (m - 1) % snap_slots
            e["snap"] = max(e["snap"], block_err(sn_np[n, sl, h], sn_ref[sl]))
        return e

    res = oracle.run_parallel(run, units, threads=threads())
    worst = {k: max(r[k] for r in res) for k in ("o", "o_64", "state", "snap")}
    return worst, res


def test_prefill_4x2048_h64_all_units(gpu):
    lens = [2048] * 4
    H = 64
    log("prefill 4x2048 H64: GPU run")
    S0 = sg.states(1, 4 * H, DEV).view(4, H, 128, 128)
    plan, cu, ins, o, st, _, _ = prefill_run("prefill_4x2048_h64", lens, H, state_in=S0)
    log("prefill 4x2048 H64: oracle on all 256 units")
    worst, _ = check_units("prefill_4x2048_h64", cu, H, [(n, h) for n in range(4) for h in range(H)], o, st, S0=np_(S0))
    log(f"prefill 4x2048 H64 worst {worst}")
    assert max(worst.values()) <= TOL


def test_prefill_gated_4x2048_h64(gpu):
    """The headline prefill with the output gated RMSNorm fused in: y bit-identical to the plain prefill
    followed by kda_gated_rmsnorm on all 524,288 (token, head) rows, the final states bit-identical, and
    two heads of y against the oracle (fp64 prefill, then the norm) at the pages' 8e-3."""
    c = synth.PREFILL_CONFIGS["prefill_4x2048_h64"]
    seed, lens, H, eps = c["seed"], c["lengths"], c["H"], 1e-6
    cu = synth.cu_seqlens(lens)
    T, N = int(cu[-1]), len(lens)
    plan = kda.kda_plan_create(cu, n_heads=H)
    ins = sg.prefill_inputs(seed, T, H, DEV)
    gate = sg.gate(seed, T, H, DEV)
    w = synth.norm_weight(seed)
    wd = torch.from_numpy(w).to(DEV)
    S0 = sg.states(seed, N * H, DEV).view(N, H, 128, 128)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
    o = torch.empty((T, H, 128), device=DEV)
    st = torch.empty((N, H, 128, 128), device=DEV)
    kda.kda_chunk_prefill(plan, *ins, st, o, ws, state_in=S0)
    y_ref = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    kda.kda_gated_rmsnorm(o, gate, wd, eps, y_ref)
    y = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    st2 = torch.empty_like(st)
    kda.kda_chunk_prefill_gated(plan, *ins, gate, wd, eps, st2, y, ws, state_in=S0)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), "fused norm differs from the unfused pair"
    assert torch.equal(st2, st)
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    worst = 0.0
    for n, h in ((0, 0), (3, 63)):
        t0 = int(cu[n])
        o_ref, _, _, _ = oracle_prefill_unit(seed, H, t0, lens[n], h, S0=np_(S0[n, h]))
        ref = oracle.gated_rmsnorm(o_ref, synth.gate_rows(seed, H, t0, lens[n], h=h), w, eps)
        yv = (yb[t0:t0 + lens[n], h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        worst = max(worst, float(np.max(np.max(np.abs(yv - ref), axis=1) / np.max(np.abs(ref), axis=1))))
    log(f"gated prefill 4x2048 H64: worst row err {worst:.2e}")
    assert worst <= 8e-3


def _row_errs(y_bits, ref):
    """Per row of 128: max |y - ref| / max |ref| (rows of ref that are exactly zero must come out zero)."""
    y = (y_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(-1, 128)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, 128)
    den = np.max(np.abs(ref), axis=1)
    err = np.max(np.abs(y - ref), axis=1)
    assert np.all(err[den == 0] == 0)
    return err[den > 0] / den[den > 0]


def test_prologue_4x2048_h64(gpu):
    """The KDA prologue at the headline prefill's size in the bench's configuration (4 x 2048 tokens,
    H = 64, conv width 4, state carried in and out): every (token, head) row of q, k, v against the
    oracle at bf16 accuracy, every beta and gk at 1e-5 relative, the carried state bit for bit."""
    rng = np.random.default_rng(2048)
    N, L, H, W, eps = 4, 2048, 64, 4, 1e-6
    lens = [L] * N
    cu = synth.cu_seqlens(lens)
    T = N * L
    xs = [synth.round_bf16(rng.standard_normal((T, H, 128))) for _ in range(3)]
    conv_w = (0.5 * rng.standard_normal((3, H * 128, W))).astype(np.float32)
    st = synth.round_bf16(rng.standard_normal((N, 3, W - 1, H * 128)))
    b = rng.standard_normal((T, H)).astype(np.float32)
    g = (2.0 * rng.standard_normal((T, H, 128))).astype(np.float32)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    outs = [torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    beta, gk = torch.empty((T, H), device=DEV), torch.empty((T, H, 128), device=DEV)
    sout = torch.empty((N, 3, W - 1, H * 128), dtype=torch.bfloat16, device=DEV)
    bf = lambda a: to_dev(a.view(np.int16)).view(torch.bfloat16)
    kda.kda_prologue(to_dev(cu.astype(np.int32)), *(bf(x) for x in xs), to_dev(conv_w), to_dev(b), to_dev(g),
                     *outs, beta, gk, conv_state_in=bf(st), conv_state_out=sout, eps=eps)
    torch.cuda.synchronize()
    got = [o.view(torch.int16).cpu().numpy().view(np.uint16) for o in outs]
    beta_h, gk_h = np_(beta), np_(gk)
    sout_h = sout.view(torch.int16).cpu().numpy().view(np.uint16)

    def one(n):
        s0 = int(cu[n])
        ref = oracle.prologue(*(x[s0:s0 + L] for x in xs), conv_w, st[n], b[s0:s0 + L], g[s0:s0 + L], eps)
        qkv = max(float(_row_errs(gt[s0:s0 + L], r).max()) for gt, r in zip(got, ref[:3]))
        eb = float(np.max(np.abs(beta_h[s0:s0 + L] - ref[3]) / np.abs(ref[3])))
        eg = float(np.max(np.abs(gk_h[s0:s0 + L] - ref[4]) / np.abs(ref[4])))
        same = np.array_equal(synth.bf16_to_f64(sout_h[n]), ref[5])
        return qkv, eb, eg, same

    res = oracle.run_parallel(one, range(N), threads=min(N, threads()))
    qkv, eb, eg = (max(r[i] for r in res) for i in range(3))
    log(f"prologue 4x2048 H64 W4: worst row err q/k/v {qkv:.2e}, beta {eb:.2e}, gk {eg:.2e}")
    assert all(r[3] for r in res), "carried state differs from the oracle's"
    assert qkv <= 5e-3 and eb <= 1e-5 and eg <= 1e-5


def test_prefill_varlen_h96_snapshots(gpu):
    H = 96
    lens = synth.prefill_lengths("varlen_h96")
    log(f"prefill varlen: {len(lens)} sequences, total {int(lens.sum())} tokens, max {int(lens.max())}")
    plan, cu, ins, o, st, snap, cnt = prefill_run("varlen_h96", lens, H, snap_slots=2)
    # counts are exact integers for every sequence
    assert np.array_equal(np_(cnt), lens // 2048)
    # longest-first and input order give the same bits
    _, _, _, o2, st2, snap2, _ = prefill_run("varlen_h96", lens, H, snap_slots=2, order=kda.KDA_PLAN_FIFO)
    assert torch.equal(o, o2) and torch.equal(st, st2) and torch.equal(snap, snap2)
    del o2, st2, snap2
    longest, shortest = int(np.argmax(lens)), int(np.argmin(lens))
    rng = np.random.default_rng(2)
    units = [(longest, h) for h in range(0, H, 3)] + [(shortest, h) for h in range(0, H, 12)]
    units += [(int(rng.integers(len(lens))), int(rng.integers(H))) for _ in range(24)]
    units = sorted(set(units))
    log(f"prefill varlen: oracle on {len(units)} units")
    worst, _ = check_units("varlen_h96", cu, H, units, o, st, snap=snap, snap_slots=2, interval=2048)
    log(f"prefill varlen worst {worst}")
    assert max(worst.values()) <= TOL


def test_ragged_verify_256x69x8(gpu):
    """The speculative-step shape with trimmed windows (1..8 tokens per request, packed back to back):
    every layer through kda_verify_ragged; the ring holds each window's raw inputs bit for bit and its
    positions past the window are untouched; the committed pool is not written; 48 sampled units
    against the oracle."""
    c = synth.VERIFY_CONFIG
    seed, B, Lyr, H, T, R = c["seed"], c["B"], c["L"], c["H"], c["T"], c["R"]
    S = B
    win = synth.trimmed_windows(seed, B, T)
    cu = np.concatenate([[0], np.cumsum(win)]).astype(np.int32)
    total = int(cu[-1])
    log(f"ragged spec step: {total} tokens over {B} requests (mean window {win.mean():.2f})")
    pool = sg.states(seed, S * Lyr * H, DEV).view(S, Lyr, H, 128, 128)
    slot_idx = torch.arange(B, dtype=torch.int32, device=DEV)
    ring_start = torch.zeros(B, dtype=torch.int32, device=DEV)
    ring = kda.Ring.empty(S, Lyr, H, R, DEV)

    def ibits(t):
        return t.view(torch.int16 if t.element_size() == 2 else torch.int32)

    for t in (ring.k, ring.v, ring.gk, ring.beta):
        ibits(t).fill_(-7)
    cu_d = torch.from_numpy(cu).to(DEV)
    # entry t < n_b of request b is packed row cu[b] + t (past the window: a valid row, masked below)
    t_idx = torch.arange(T)
    n_b = torch.from_numpy(win)
    valid = (t_idx[None, :] < n_b[:, None]).to(DEV)
    rows = (torch.from_numpy(cu[:-1]).long()[:, None] + torch.minimum(t_idx[None, :], n_b[:, None] - 1)).to(DEV)
    rng = np.random.default_rng(5)
    samples = sorted({(int(rng.integers(B)), int(rng.integers(Lyr)), int(rng.integers(H))) for _ in range(48)})
    o_s = {}
    for l in range(Lyr):
        ins = sg.prefill_inputs(seed, total, H, DEV, sub=l)
        o = torch.empty((total, H, 128), device=DEV)
        kda.kda_verify_ragged(*ins, cu_d, pool, slot_idx, o, layer=l, max_tok=T, ring=ring, ring_start=ring_start)
        for src, rt in ((ins[1], ring.k), (ins[2], ring.v), (ins[3], ring.gk)):
            want = ibits(src)[rows].permute(0, 2, 1, 3)  # [B, H, T, 128]
            got = ibits(rt[:, l, :, :T])
            m = valid[:, None, :, None]
            assert torch.equal(torch.where(m, got, 0), torch.where(m, want, 0)), f"ring entries differ at layer {l}"
            assert bool(torch.all(torch.where(m, -7, got) == -7)), f"ring written past a window at layer {l}"
        want = ibits(ins[4])[rows].permute(0, 2, 1)
        got = ibits(ring.beta[:, l, :, :T])
        assert torch.equal(torch.where(valid[:, None, :], got, 0), torch.where(valid[:, None, :], want, 0))
        assert bool(torch.all(torch.where(valid[:, None, :], -7, got) == -7))
        for (b, ll, h) in samples:
            if ll == l:
                o_s[(b, ll, h)] = np_(o[int(cu[b]):int(cu[b + 1]), h])
    torch.cuda.synchronize()
    fresh = sg.states(seed, S * Lyr * H, DEV).view(S, Lyr, H, 128, 128)
    assert torch.equal(pool, fresh), "verify wrote the committed state"
    del fresh

    def run(u):
        b, l, h = u
        q, k, v, gk, beta = synth.prefill_rows(seed, H, int(cu[b]), int(win[b]), h=h, sub=l)
        S0 = synth.state_rows(seed, (b * Lyr + l) * H + h, 1)[0]
        o_ref, _, _ = oracle.verify(q, k, v, gk, beta, S0)
        return block_err(o_s[u], o_ref)

    worst = max(oracle.run_parallel(run, samples, threads=threads()))
    log(f"ragged spec step worst {worst:.2e}")
    assert worst <= TOL


def test_spec_step_256x69x8(gpu):
    c = synth.VERIFY_CONFIG
    seed, B, Lyr, H, T, R = c["seed"], c["B"], c["L"], c["H"], c["T"], c["R"]
    S = B
    log("spec step: generating the committed pool and inputs")
    pool = sg.states(seed, S * Lyr * H, DEV).view(S, Lyr, H, 128, 128)
    acc_np = synth.geometric_accept(seed, B)
    acc = torch.from_numpy(acc_np).to(torch.int32).to(DEV)
    slot_idx = torch.arange(B, dtype=torch.int32, device=DEV)
    ring_start = torch.zeros(B, dtype=torch.int32, device=DEV)
    ring = kda.Ring.empty(S, Lyr, H, R, DEV)
    commit = torch.empty_like(pool)
    rng = np.random.default_rng(3)
    samples = sorted({(int(rng.integers(B)), int(rng.integers(Lyr)), int(rng.integers(H))) for _ in range(48)})
    o_s, o_c = {}, {}
    gap = 0.0  # served (chunked) outputs against the token-by-token ones, every unit, normwise per unit
    for l in range(Lyr):
        ins = sg.prefill_inputs(seed, B * T, H, DEV, sub=l)
        # the speculative step as served: no recurrent commit (the chunked matrix-core path) ...
        o = torch.empty((B * T, H, 128), device=DEV)
        kda.kda_verify(*ins, pool, slot_idx, o, layer=l, n_tok=T, ring=ring, ring_start=ring_start)
        # ... and with the recurrent commit the fold is compared against (the token-by-token path)
        oc = torch.empty((B * T, H, 128), device=DEV)
        kda.kda_verify(*ins, pool, slot_idx, oc, layer=l, n_tok=T, ring=ring, ring_start=ring_start, commit_len=acc,
                       commit_pool=commit)
        # the ring holds the raw inputs of every request at positions 0..T-1, bit for bit
        k_in = ins[1].view(B, T, H, 128).permute(0, 2, 1, 3)
        v_in = ins[2].view(B, T, H, 128).permute(0, 2, 1, 3)
        g_in = ins[3].view(B, T, H, 128).permute(0, 2, 1, 3)
        b_in = ins[4].view(B, T, H).permute(0, 2, 1)
        assert torch.equal(ring.k[:, l, :, :T], k_in) and torch.equal(ring.v[:, l, :, :T], v_in)
        assert torch.equal(ring.gk[:, l, :, :T], g_in) and torch.equal(ring.beta[:, l, :, :T], b_in)
        for (b, ll, h) in samples:
            if ll == l:
                o_s[(b, ll, h)] = np_(o.view(B, T, H, 128)[b, :, h])
                o_c[(b, ll, h)] = np_(oc.view(B, T, H, 128)[b, :, h])
        d = (o - oc).abs().view(B, T, H, 128).amax(dim=(1, 3)) / oc.abs().view(B, T, H, 128).amax(dim=(1, 3))
        gap = max(gap, float(d.max()))
    torch.cuda.synchronize()
    # verify never wrote the committed pool
    fresh = sg.states(seed, S * Lyr * H, DEV).view(S, Lyr, H, 128, 128)
    assert torch.equal(pool, fresh)
    del fresh
    log("spec step: fold")
    kda.kda_replay_fold(pool, slot_idx, ring, acc, ring_start=ring_start)
    torch.cuda.synchronize()
    # bit-identical to verify's recurrent commit on every (request, layer, head)
    assert torch.equal(pool, commit), "fold differs from the recurrent commit"
    log(f"spec step: oracle on {len(samples)} units")
    pool_np = {u: np_(pool[u[0], u[1], u[2]]) for u in samples}

    def run(u):
        b, l, h = u
        q, k, v, gk, beta = synth.prefill_rows(seed, H, b * T, T, h=h, sub=l)
        S0 = synth.state_rows(seed, (b * Lyr + l) * H + h, 1)[0]
        o_ref, Sc, _ = oracle.verify(q, k, v, gk, beta, S0, commit_len=int(acc_np[b]))
        return max(block_err(o_s[u], o_ref), block_err(o_c[u], o_ref), block_err(pool_np[u], Sc))

    worst = max(oracle.run_parallel(run, samples, threads=threads()))
    log(f"spec step worst {worst:.2e}; chunked vs token-by-token outputs, worst of all "
        f"{B * Lyr * H} units: {gap:.2e}")
    assert worst <= TOL and gap <= TOL

    # The next step through the fused path: kda_fold_verify per layer folds this step's window
    # (positions 0..T-1, accepted lengths acc) into a fresh copy of the committed pool and verifies
    # the next window (positions T..2T-1) from it; it must equal the fold above followed by a
    # verify of the next window from the folded pool, bit for bit.
    log("spec step: next step, fused fold-then-verify against fold + verify")
    ring_next = torch.full((B,), T, dtype=torch.int32, device=DEV)
    ring_f = kda.Ring(ring.k.clone(), ring.v.clone(), ring.gk.clone(), ring.beta.clone())
    pool_f = sg.states(seed, S * Lyr * H, DEV).view(S, Lyr, H, 128, 128)
    for l in range(Lyr):
        ins2 = sg.prefill_inputs(seed, B * T, H, DEV, sub=Lyr + l)
        o_ref = torch.empty((B * T, H, 128), device=DEV)
        kda.kda_verify(*ins2, pool, slot_idx, o_ref, layer=l, n_tok=T, ring=ring, ring_start=ring_next)
        o_f = torch.empty((B * T, H, 128), device=DEV)
        kda.kda_fold_verify(*ins2, pool_f, slot_idx, o_f, layer=l, n_tok=T, ring=ring_f, fold_len=acc,
                            fold_start=ring_start, ring_start=ring_next)
        assert torch.equal(o_f, o_ref), f"fused fold-then-verify output differs at layer {l}"
    torch.cuda.synchronize()
    assert torch.equal(pool_f, pool), "fused fold differs from the fold"
    for a, b in ((ring_f.k, ring.k), (ring_f.v, ring.v), (ring_f.gk, ring.gk), (ring_f.beta, ring.beta)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_long_context_1m_then_decode(gpu):
    H, T = 96, 1048576
    cfg = synth.PREFILL_CONFIGS["long_1m_h96"]
    seed = cfg["seed"]
    log("long context: generating 1M x 96 inputs on the device")
    # 96 (sequence, head) chains for 256 compute units: the automatic plan splits each into two
    # value blocks; the whole-chain plan must give the same bits
    plan, cu, ins, o, st, snap, cnt = prefill_run("long_1m_h96", [T], H, snap_slots=2, v_blocks=0)
    assert int(cnt[0]) == T // 4096
    heads = [7, 60]
    o_np = {h: np_(o[:, h]) for h in heads}
    st_split, snap_split = st.clone(), snap.clone()
    whole = kda.kda_plan_create(cu, n_heads=H, snap_interval=4096, v_blocks=1)
    ms = prefill_launch(whole, ins, o, st, snap, cnt, 2)
    log(f"long context: whole-chain plan ({kda.kda_plan_num_items(whole)} items) {ms:.2f} ms")
    assert torch.equal(st, st_split) and torch.equal(snap, snap_split)
    for h in heads:
        assert np.array_equal(np_(o[:, h]), o_np[h])
    del ins, o, st_split, snap_split
    torch.cuda.empty_cache()
    # 128 single-token decode steps from the final state: verify with n_tok = 1 and an in-place commit
    pool = st.view(1, 1, H, 128, 128).clone()
    slot = torch.zeros(1, dtype=torch.int32, device=DEV)
    one = torch.ones(1, dtype=torch.int32, device=DEV)
    dec_tids = (synth.T_DEC_Q, synth.T_DEC_K, synth.T_DEC_V, synth.T_DEC_GK, synth.T_DEC_BETA)
    dq, dk, dv, dg, db = sg.prefill_inputs(seed, synth.DECODE_STEPS, H, DEV, tids=dec_tids)
    dec_o = torch.empty((synth.DECODE_STEPS, H, 128), device=DEV)
    for t in range(synth.DECODE_STEPS):
        kda.kda_verify(dq[t:t + 1], dk[t:t + 1], dv[t:t + 1], dg[t:t + 1], db[t:t + 1], pool, slot,
                       dec_o[t:t + 1], layer=0, n_tok=1, commit_len=one, commit_pool=pool)
    torch.cuda.synchronize()
    st_np, sn_np, dec_np, fin_np = np_(st), np_(snap), np_(dec_o), np_(pool[0, 0])
    log(f"long context: oracle on heads {heads} (1,048,576 tokens each) and their decode steps")

    def run(h):
        o_ref, S_ref, sn_ref, c = oracle_prefill_unit(seed, H, 0, T, h, snap_interval=4096, snap_slots=2)
        e = {"o": block_err(o_np[h], o_ref), "o_64": rows_err(o_np[h], o_ref, 64), "state": block_err(st_np[0, h], S_ref),
             "snap": max(block_err(sn_np[0, s, h], sn_ref[s]) for s in range(2))}
        q, k, v, gk, beta = synth.prefill_rows(seed, H, 0, synth.DECODE_STEPS, h=h, tids=dec_tids)
        do_ref, dS_ref, _, _ = oracle.recurrent(q, k, v, gk, beta, S_ref)
        e["decode_o"] = block_err(dec_np[:, h], do_ref)
        e["decode_state"] = block_err(fin_np[h], dS_ref)
        return e

    res = oracle.run_parallel(run, heads, threads=len(heads))
    worst = {k: max(r[k] for r in res) for k in res[0]}
    log(f"long context worst {worst}")
    assert max(worst.values()) <= TOL
