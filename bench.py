"""Benchmark of the KDA hot path on one MI355X.

Headline (``value``): chunked-prefill throughput in tokens*heads/s on the
workload "4 sequences x 2048 tokens, H = 64, K = V = 128, bf16 q/k/v, fp32
gk/beta/state, state_in ~ N(0, 0.1^2)". One step = one kda_chunk_prefill call
with the work list resident (one persistent-kernel launch), timed with HIP
events on the launch stream. Beside it, in the same JSON line:

* ``verify_fold``: one speculative step of the workload "256 requests x 69
  layers x 8 heads, gamma + 1 = 8 bf16 draft tokens, ring length 16, accepted
  lengths geometric (mean 2.7, clipped to [1, 8])" = 69 kda_verify launches +
  one kda_replay_fold launch, in us/step (committed states restored from a
  pristine copy outside the timed region before every step); beside it the
  same step through kda_fold_verify, and the verify with trimmed windows
  (1..8 tokens per request, packed) through kda_verify_ragged;
* ``prefill_gated_norm``: the same prefill with the output gated RMSNorm,
  fused into its epilogue (kda_chunk_prefill_gated) and unfused (the prefill,
  then kda_gated_rmsnorm over its fp32 output);
* ``prologue``: the step before the recurrence (kda_prologue) over the same
  tokens, in us and GB/s;
* ``roofline``: HBM roofline of the prefill kernel (algorithmic bytes per
  launch / measured launch time, against 8 TB/s);
* ``cpu_baseline``: the fp64 oracle (token-by-token) timed on this host's
  cores over the same prefill workload.

Inputs are synthetic, generated on the device by the seeded generator.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "KDA prefill tokens*heads/s and verify+fold us/step at 1 GPU; % of roofline"

# HBM bytes per prefill launch measured by rocprofv3 PMC (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000, the
# factors that make a plain 1 GiB copy read 1 GiB and write 1 GiB); set to None whenever the kernel
# changes until it is measured again
PREFILL_TRAFFIC_BYTES = 980_824_721


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--vf-steps", type=int, default=5, help="timed verify+fold steps")
    ap.add_argument("--no-verify-fold", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill (for profilers)")
    ap.add_argument("--verify-fold-only", action="store_true", help="time only the speculative step (for profilers)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy, the reference kernel for scaling HBM byte counters")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_bytes(n_seq, L, H, with_state_in=True):
    """Algorithmic HBM bytes of one prefill launch: per token*head q,k,v bf16 (3*256) + gk fp32 (512)
    + beta (4) + o fp32 (512) = 1,796 B; per (sequence, head) 64 KiB state out (+ 64 KiB in)."""
    th = n_seq * L * H
    st = n_seq * H * 65536 * (2 if with_state_in else 1)
    return th * 1796 + st


def settle(step, torch, seconds=0.25):
    """Run the step untimed until `seconds` of wall time have passed: the GPU's clocks ramp up
    over the first ~100 launches of a short kernel, and the timed region should see the steady
    state. This precedes the W warm-up steps and is never part of the timed region."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()


def bench_prefill(args, torch, kda, sg, synth):
    dev = "cuda:0"
    N, L, H = 4, 2048, 64
    cfg = synth.PREFILL_CONFIGS["prefill_4x2048_h64"]
    seed = cfg["seed"]
    cu = synth.cu_seqlens([L] * N)
    T = int(cu[-1])
    q, k, v, gk, beta = sg.prefill_inputs(seed, T, H, dev)
    S0 = sg.states(seed, N * H, dev).view(N, H, 128, 128)
    o = torch.empty((T, H, 128), device=dev)
    st = torch.empty((N, H, 128, 128), device=dev)
    plan = kda.kda_plan_create(cu, n_heads=H)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=dev)
    kda.kda_plan_upload(plan, ws)
    flags = kda.KDA_PREFILL_PLAN_RESIDENT

    def step():
        kda.kda_chunk_prefill(plan, q, k, v, gk, beta, st, o, ws, state_in=S0, flags=flags)

    settle(step, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tokens_heads = N * L * H
    byts = prefill_bytes(N, L, H)
    achieved = byts / (ms * 1e-3) / 1e9
    res = dict(ms=ms, value=tokens_heads / (ms * 1e-3), bytes=byts, achieved=achieved, N=N, L=L, H=H)
    del q, k, v, gk, beta, o, st, S0
    return res


def bench_prefill_gated(args, torch, kda, sg, synth):
    """The headline prefill with the output gated RMSNorm: fused (kda_chunk_prefill_gated, bf16 y) against
    the same two steps unfused (kda_chunk_prefill, then kda_gated_rmsnorm over its fp32 o)."""
    dev = "cuda:0"
    N, L, H = 4, 2048, 64
    seed = synth.PREFILL_CONFIGS["prefill_4x2048_h64"]["seed"]
    cu = synth.cu_seqlens([L] * N)
    T = int(cu[-1])
    q, k, v, gk, beta = sg.prefill_inputs(seed, T, H, dev)
    gate = sg.gate(seed, T, H, dev)
    w = torch.from_numpy(synth.norm_weight(seed)).to(dev)
    S0 = sg.states(seed, N * H, dev).view(N, H, 128, 128)
    o = torch.empty((T, H, 128), device=dev)
    y = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    st = torch.empty((N, H, 128, 128), device=dev)
    plan = kda.kda_plan_create(cu, n_heads=H)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=dev)
    kda.kda_plan_upload(plan, ws)
    flags = kda.KDA_PREFILL_PLAN_RESIDENT
    eps = 1e-6

    def fused():
        kda.kda_chunk_prefill_gated(plan, q, k, v, gk, beta, gate, w, eps, st, y, ws, state_in=S0, flags=flags)

    def unfused():
        kda.kda_chunk_prefill(plan, q, k, v, gk, beta, st, o, ws, state_in=S0, flags=flags)
        kda.kda_gated_rmsnorm(o, gate, w, eps, y)

    stream = torch.cuda.current_stream()
    res = {}
    for name, step in (("fused", fused), ("unfused", unfused)):
        settle(step, torch)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / args.steps
    th = N * L * H
    st_b = N * H * 65536 * 2
    # fused: q, k, v, gate bf16 + gk fp32 + beta + y bf16 = 1,796 B per token*head; unfused adds the norm's
    # own pass (o fp32 read, gate read, y written) on top of the plain prefill's 1,796 B
    fused_b, unfused_b = th * 1796 + st_b, th * (1796 + 1024) + st_b
    del q, k, v, gk, beta, gate, o, y, st, S0
    return dict(fused_ms=res["fused"], unfused_ms=res["unfused"], fused_bytes=fused_b, unfused_bytes=unfused_b,
                tokens_heads=th)


def bench_prologue(args, torch, kda, sg, synth):
    """The KDA prologue (short conv width 4 + SiLU with the state carry, q/k L2 norm, beta sigmoid,
    gk = -softplus) over the headline prefill's tokens: one kda_prologue launch."""
    import numpy as np

    dev = "cuda:0"
    N, L, H, W = 4, 2048, 64, 4
    seed = synth.PREFILL_CONFIGS["prefill_4x2048_h64"]["seed"]
    cu = torch.from_numpy(synth.cu_seqlens([L] * N).astype(np.int32)).to(dev)
    T = N * L
    g = torch.Generator(device=dev).manual_seed(seed)
    xs = [torch.randn((T, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(3)]
    conv_w = 0.5 * torch.randn((3, H * 128, W), generator=g, device=dev)
    st_in = torch.randn((N, 3, W - 1, H * 128), generator=g, device=dev).to(torch.bfloat16)
    st_out = torch.empty_like(st_in)
    b_raw = torch.randn((T, H), generator=g, device=dev)
    g_raw = torch.randn((T, H, 128), generator=g, device=dev)
    outs = [torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    beta, gk = torch.empty((T, H), device=dev), torch.empty((T, H, 128), device=dev)

    def step():
        kda.kda_prologue(cu, *xs, conv_w, b_raw, g_raw, *outs, beta, gk, conv_state_in=st_in, conv_state_out=st_out)

    settle(step, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # per token*head: x_q, x_k, x_v bf16 in (768) + g_raw (512) + b_raw (4); q, k, v bf16 out (768) + gk (512)
    # + beta (4) = 2,568 B; plus the carried state in and out
    byts = T * H * 2568 + 2 * N * 3 * (W - 1) * H * 128 * 2
    del xs, conv_w, st_in, st_out, b_raw, g_raw, outs, beta, gk
    return dict(ms=ms, bytes=byts, gbs=byts / (ms * 1e-3) / 1e9)


def bench_state_moves(args, torch, kda, sg, synth):
    """The prefix-cache snapshot of the speculative step's batch: 256 requests, each a slot of 69 layers x
    8 heads of 128 x 128 fp32 state (36.2 MB), copied working -> fresh slot in one kda_state_move launch;
    the moves come from the host slot protocol (SlotPool.open, then snapshot per request)."""
    dev = "cuda:0"
    c = synth.VERIFY_CONFIG
    B, Lyr, H = c["B"], c["L"], c["H"]
    slots = kda.SlotPool(2 * B)
    pool = torch.zeros((2 * B, Lyr, H, 128, 128), device=dev)
    reqs = [slots.open()[0] for _ in range(B)]
    moves = torch.tensor([slots.snapshot(r) for r in reqs], dtype=torch.int32, device=dev)
    flat = pool.view(2 * B, -1)

    def step():
        kda.kda_state_move(flat, moves)

    settle(step, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    byts = 2 * B * Lyr * H * 65536
    del pool, flat
    return dict(ms=ms, bytes=byts, gbs=byts / (ms * 1e-3) / 1e9)


def bench_long_context(args, torch, kda, sg, synth):
    """The long-context workload: one 1,048,576-token sequence x 96 heads through kda_chunk_prefill (the
    automatic plan: 192 half-chains; snapshots every 4096 tokens into 2 slots), then 128 single-token
    decode steps from its final state (kda_verify, n_tok = 1, commit in place), launched one by one and
    as one replayed HIP graph."""
    dev = "cuda:0"
    c = synth.PREFILL_CONFIGS["long_1m_h96"]
    seed, H, T = c["seed"], c["H"], sum(c["lengths"])
    torch.cuda.empty_cache()  # about 180 GB of inputs and outputs follow
    cu = synth.cu_seqlens([T])
    plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=c["snap_interval"], v_blocks=0)
    ins = sg.prefill_inputs(seed, T, H, dev)
    o = torch.empty((T, H, 128), device=dev)
    st = torch.empty((1, H, 128, 128), device=dev)
    slots = c["snap_slots"]
    snap = torch.empty((1, slots, H, 128, 128), device=dev)
    cnt = torch.empty((1,), dtype=torch.int32, device=dev)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=dev)
    kda.kda_plan_upload(plan, ws)

    def step():
        kda.kda_chunk_prefill(plan, *ins, st, o, ws, snap=snap, snap_slots=slots, snap_count=cnt,
                              flags=kda.KDA_PREFILL_PLAN_RESIDENT)

    n = max(1, min(args.steps, 3))
    step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    byts = prefill_bytes(1, T, H, with_state_in=False) + (T // c["snap_interval"]) * H * 65536
    del ins, o
    torch.cuda.empty_cache()
    # decode
    steps = synth.DECODE_STEPS
    tids = (synth.T_DEC_Q, synth.T_DEC_K, synth.T_DEC_V, synth.T_DEC_GK, synth.T_DEC_BETA)
    dq, dk, dv, dg, db = sg.prefill_inputs(seed, steps, H, dev, tids=tids)
    pool = st.view(1, 1, H, 128, 128).clone()
    slot = torch.zeros(1, dtype=torch.int32, device=dev)
    one = torch.ones(1, dtype=torch.int32, device=dev)
    dec_o = torch.empty((steps, H, 128), device=dev)

    def decode():
        for t in range(steps):
            kda.kda_verify(dq[t:t + 1], dk[t:t + 1], dv[t:t + 1], dg[t:t + 1], db[t:t + 1], pool, slot,
                           dec_o[t:t + 1], layer=0, n_tok=1, commit_len=one, commit_pool=pool)

    def timed(fn, reps):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * steps)

    decode()
    eager_us = timed(decode, 5)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        decode()
    g.replay()
    graph_us = timed(g.replay, 5)
    dec_bytes = H * (2 * 65536 + 1796)
    # a whole decode layer from the projections: prologue + step + gated RMSNorm, as three launches per
    # step (kda_prologue, kda_verify, kda_gated_rmsnorm) and as one (kda_decode), both replayed as graphs
    W = 4
    gen = torch.Generator(device=dev).manual_seed(seed)
    xs = [torch.randn((steps, H, 128), generator=gen, device=dev).to(torch.bfloat16) for _ in range(3)]
    conv_w = 0.5 * torch.randn((3, H * 128, W), generator=gen, device=dev)
    cst = [torch.randn((1, 3, W - 1, H * 128), generator=gen, device=dev).to(torch.bfloat16) for _ in range(2)]
    b_raw = torch.randn((steps, H), generator=gen, device=dev)
    g_raw = torch.randn((steps, H, 128), generator=gen, device=dev)
    gate = torch.randn((steps, H, 128), generator=gen, device=dev).to(torch.bfloat16)
    norm_w = 1.0 + 0.1 * torch.randn((128,), generator=gen, device=dev)
    y = torch.empty((steps, H, 128), dtype=torch.bfloat16, device=dev)
    q, k, v = (torch.empty((1, H, 128), dtype=torch.bfloat16, device=dev) for _ in range(3))
    beta, gk, o1 = torch.empty((1, H), device=dev), torch.empty((1, H, 128), device=dev), torch.empty((1, H, 128), device=dev)
    cu1 = torch.tensor([0, 1], dtype=torch.int32, device=dev)

    def chain():
        for t in range(steps):
            kda.kda_prologue(cu1, xs[0][t:t + 1], xs[1][t:t + 1], xs[2][t:t + 1], conv_w, b_raw[t:t + 1],
                             g_raw[t:t + 1], q, k, v, beta, gk, conv_state_in=cst[t & 1], conv_state_out=cst[1 - (t & 1)])
            kda.kda_verify(q, k, v, gk, beta, pool, slot, o1, layer=0, n_tok=1, commit_len=one, commit_pool=pool)
            kda.kda_gated_rmsnorm(o1, gate[t:t + 1], norm_w, 1e-6, y[t:t + 1])

    def fused():
        for t in range(steps):
            kda.kda_decode(xs[0][t:t + 1], xs[1][t:t + 1], xs[2][t:t + 1], conv_w, cst[0], b_raw[t:t + 1],
                           g_raw[t:t + 1], pool, slot, gate[t:t + 1], norm_w, y[t:t + 1])

    graphs = {}
    for name, fn in (("chain", chain), ("fused", fused)):
        fn()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        gr.replay()
        graphs[name] = timed(gr.replay, 5)
    return dict(ms=ms, bytes=byts, gbs=byts / (ms * 1e-3) / 1e9, T=T, H=H, items=kda.kda_plan_num_items(plan),
                eager_us=eager_us, graph_us=graph_us, dec_gbs=dec_bytes / (graph_us * 1e-6) / 1e9,
                layer_chain_us=graphs["chain"], layer_fused_us=graphs["fused"])


def bench_verify_fold(args, torch, kda, sg, synth):
    dev = "cuda:0"
    c = synth.VERIFY_CONFIG
    seed, B, Lyr, H, T, R = c["seed"], c["B"], c["L"], c["H"], c["T"], c["R"]
    S = B
    pool = sg.states(seed, S * Lyr * H, dev).view(S, Lyr, H, 128, 128)
    pristine = pool.clone()
    ring = kda.Ring.empty(S, Lyr, H, R, dev)
    ins = [sg.prefill_inputs(seed, B * T, H, dev, sub=l) for l in range(Lyr)]
    slot_idx = torch.arange(B, dtype=torch.int32, device=dev)
    ring_start = torch.zeros(B, dtype=torch.int32, device=dev)
    acc = torch.from_numpy(synth.geometric_accept(seed, B)).to(torch.int32).to(dev)
    o = torch.empty((B * T, H, 128), device=dev)
    stream = torch.cuda.current_stream()

    def one_step(times):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        for l in range(Lyr):
            q, k, v, gk, beta = ins[l]
            kda.kda_verify(q, k, v, gk, beta, pool, slot_idx, o, layer=l, n_tok=T, ring=ring, ring_start=ring_start)
        ev[1].record(stream)
        kda.kda_replay_fold(pool, slot_idx, ring, acc, ring_start=ring_start)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if times is not None:
            times.append((ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])))

    def untimed():
        pool.copy_(pristine)
        one_step(None)

    settle(untimed, torch)
    for _ in range(max(1, args.warmup // 2)):
        untimed()
    times = []
    for _ in range(args.vf_steps):
        pool.copy_(pristine)  # the fold advances states in place: restore outside the timed region
        torch.cuda.synchronize()
        one_step(times)
    ver = sum(t[0] for t in times) / len(times)
    fol = sum(t[1] for t in times) / len(times)

    # The same step through the fused path: one kda_fold_verify per layer folds the window the
    # verifies above recorded (positions 0..T-1, the accepted lengths) into the committed state and
    # verifies the next window (positions T..2T-1) from it.
    ring_next = torch.full((B,), T, dtype=torch.int32, device=dev)

    def fused_step(times):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for l in range(Lyr):
            q, k, v, gk, beta = ins[l]
            kda.kda_fold_verify(q, k, v, gk, beta, pool, slot_idx, o, layer=l, n_tok=T, ring=ring, fold_len=acc,
                                fold_start=ring_start, ring_start=ring_next)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if times is not None:
            times.append(ev[0].elapsed_time(ev[1]))

    for _ in range(max(1, args.warmup // 2)):
        pool.copy_(pristine)
        fused_step(None)
    ftimes = []
    for _ in range(args.vf_steps):
        pool.copy_(pristine)
        torch.cuda.synchronize()
        fused_step(ftimes)
    fus = sum(ftimes) / len(ftimes)

    # The verify with trimmed windows: request b keeps n_b of its 8 draft tokens (1..8), packed back to
    # back; one kda_verify_ragged per layer. The committed pool is only read.
    import numpy as np

    win = synth.trimmed_windows(seed, B, T)
    cu_r = np.concatenate([[0], np.cumsum(win)]).astype(np.int32)
    tot_r = int(cu_r[-1])
    del ins
    ins_r = [sg.prefill_inputs(seed, tot_r, H, dev, sub=l) for l in range(Lyr)]
    cu_d = torch.from_numpy(cu_r).to(dev)
    o_r = torch.empty((tot_r, H, 128), device=dev)

    def ragged_step(times):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for l in range(Lyr):
            kda.kda_verify_ragged(*ins_r[l], cu_d, pool, slot_idx, o_r, layer=l, max_tok=T, ring=ring,
                                  ring_start=ring_start)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if times is not None:
            times.append(ev[0].elapsed_time(ev[1]))

    for _ in range(max(1, args.warmup // 2)):
        ragged_step(None)
    rtimes = []
    for _ in range(args.vf_steps):
        ragged_step(rtimes)
    rag = sum(rtimes) / len(rtimes)
    units = S * Lyr * H
    acc_mean = float(acc.float().mean())
    v_bytes = units * (65536 + T * (768 + 512 + 4 + 512 + 1028))  # state + inputs + o + ring entries
    f_bytes = units * (2 * 65536) + int(round(float(acc.float().sum()) * Lyr * H * 1028))
    # fused: the state read once, written back, the folded entries read, the verify's inputs and outputs
    fv_bytes = units * (2 * 65536 + T * (768 + 512 + 4 + 512 + 1028)) + int(round(float(acc.float().sum()) * Lyr * H * 1028))
    r_bytes = units * 65536 + tot_r * Lyr * H * (768 + 512 + 4 + 512 + 1028)
    res = dict(verify_ms=ver, fold_ms=fol, accept_mean=acc_mean,
               verify_gbs=v_bytes / (ver * 1e-3) / 1e9, fold_gbs=f_bytes / (fol * 1e-3) / 1e9,
               verify_bytes=v_bytes, fold_bytes=f_bytes, fused_ms=fus, fused_bytes=fv_bytes,
               fused_gbs=fv_bytes / (fus * 1e-3) / 1e9, ragged_ms=rag, ragged_bytes=r_bytes,
               ragged_gbs=r_bytes / (rag * 1e-3) / 1e9, ragged_mean_window=float(win.mean()))
    del pool, pristine, ring, ins_r, o, o_r
    return res


def cpu_baseline(synth, oracle):
    """The fp64 oracle, as it is, on this host's cores: every (sequence, head) unit of the
    prefill workload (4 x 2048 tokens x 64 heads). Input generation is not timed."""
    N, L, H = 4, 2048, 64
    seed = synth.PREFILL_CONFIGS["prefill_4x2048_h64"]["seed"]
    threads = min(16, os.cpu_count() or 1)
    units = [(n, h) for n in range(N) for h in range(H)]
    data = {}
    for n, h in units:
        q, k, v, gk, beta = synth.prefill_rows(seed, H, n * L, L, h=h)
        S0 = synth.state_rows(seed, n * H + h, 1)[0]
        data[(n, h)] = (oracle.f64(q), oracle.f64(k), oracle.f64(v), oracle.f64(gk), oracle.f64(beta), S0)

    def run(u):
        q, k, v, gk, beta, S0 = data[u]
        oracle.recurrent(q, k, v, gk, beta, S0)

    t0 = time.perf_counter()
    oracle.run_parallel(run, units, threads=threads)
    dt = time.perf_counter() - t0
    return dict(value=N * L * H / dt, unit="tokens*heads/s", cores=threads, kind="oracle",
                sample=f"full workload: {N} x {L} tokens x {H} heads (fp64 token-by-token), {dt:.2f} s wall")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the units of work are "
              f"independent and need no collectives; one GPU's share is what is measured)", file=sys.stderr)
        sys.exit(2)
    import torch

    import linear_attention_recurrence_amd as kda
    import synth
    import synth.gpu as sg

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()
    if args.verify_fold_only:
        vf = bench_verify_fold(args, torch, kda, sg, synth)
        print(json.dumps({"verify_us": vf["verify_ms"] * 1e3, "fold_us": vf["fold_ms"] * 1e3,
                          "verify_gbs": vf["verify_gbs"], "fold_gbs": vf["fold_gbs"],
                          "fused_us": vf["fused_ms"] * 1e3, "fused_gbs": vf["fused_gbs"],
                          "ragged_verify_us": vf["ragged_ms"] * 1e3, "ragged_gbs": vf["ragged_gbs"]}), flush=True)
        return
    log("prefill: generating inputs and timing")
    pf = bench_prefill(args, torch, kda, sg, synth)
    log(f"prefill: {pf['ms'] * 1e3:.1f} us/launch, {pf['achieved']:.0f} GB/s")
    pg = None
    if not args.prefill_only:
        log("prefill with the output gated RMSNorm: fused and unfused")
        pg = bench_prefill_gated(args, torch, kda, sg, synth)
    pro = None
    if not args.prefill_only:
        log("prologue")
        pro = bench_prologue(args, torch, kda, sg, synth)
    mvs = None
    if not args.prefill_only:
        log("state moves")
        mvs = bench_state_moves(args, torch, kda, sg, synth)
    lc = None
    if not args.prefill_only:
        log("long context: 1M x 96 prefill, then 128 decode steps")
        try:
            lc = bench_long_context(args, torch, kda, sg, synth)
        except torch.cuda.OutOfMemoryError as e:  # the headline line must still be printed
            log(f"long context skipped: {e}")
            torch.cuda.empty_cache()
    vf = None
    if not (args.no_verify_fold or args.prefill_only):
        log("verify+fold: generating inputs and timing")
        vf = bench_verify_fold(args, torch, kda, sg, synth)
        log(f"verify+fold: {vf['verify_ms'] * 1e3:.0f} + {vf['fold_ms'] * 1e3:.0f} us; fused {vf['fused_ms'] * 1e3:.0f} us")
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies (1 GiB read + 1 GiB written each)")
        del src, dst
    cpu = None
    if not (args.no_cpu_baseline or args.prefill_only):
        import oracle

        log("cpu baseline: fp64 oracle on host cores")
        cpu = cpu_baseline(synth, oracle)
    traffic = PREFILL_TRAFFIC_BYTES
    line = {
        "metric": METRIC,
        "value": pf["value"],
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "chunked prefill: 4 sequences x 2048 tokens, H=64, K=V=128, bf16 q/k/v, "
                               "fp32 gk/beta/state, state_in N(0,0.1^2), chunk 32, one persistent launch",
                   "n_seq": pf["N"], "seq_len": pf["L"], "heads": pf["H"], "head_dim": 128},
        "roofline": {"bound": "hbm", "achieved": pf["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pf["achieved"] / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "kda::prefill_kernel<false>", "algorithmic_bytes_per_launch": pf["bytes"]},
        "cpu_baseline": cpu,
    }
    if pg is not None:
        line["prefill_gated_norm"] = {
            "fused_us": pg["fused_ms"] * 1e3, "unfused_us": pg["unfused_ms"] * 1e3,
            "fused_tokens_heads_per_s": pg["tokens_heads"] / (pg["fused_ms"] * 1e-3),
            "fused_gbs": pg["fused_bytes"] / (pg["fused_ms"] * 1e-3) / 1e9,
            "fused_hbm_frac": pg["fused_bytes"] / (pg["fused_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "workload": "the headline prefill followed by the output gated RMSNorm (gate N(0,1) bf16, weights "
                        "1 + 0.1 N(0,1), eps 1e-6, bf16 y): kda_chunk_prefill_gated vs kda_chunk_prefill + "
                        "kda_gated_rmsnorm",
        }
    if pro is not None:
        line["prologue"] = {
            "us": pro["ms"] * 1e3, "gbs": pro["gbs"], "hbm_frac": pro["gbs"] / HBM_PEAK_GBS,
            "workload": "kda_prologue over the headline prefill's 8,192 tokens x 64 heads: conv width 4 with the "
                        "state carried in and out, SiLU, q/k L2 norm, beta sigmoid, gk = -softplus (2,568 B per "
                        "token*head)",
        }
    if lc is not None:
        line["long_context"] = {
            "prefill_ms": lc["ms"], "prefill_tokens_heads_per_s": lc["T"] * lc["H"] / (lc["ms"] * 1e-3),
            "prefill_gbs": lc["gbs"], "prefill_hbm_frac": lc["gbs"] / HBM_PEAK_GBS, "prefill_items": lc["items"],
            "decode_us_per_step_eager": lc["eager_us"], "decode_us_per_step_graph": lc["graph_us"],
            "decode_gbs_graph": lc["dec_gbs"], "decode_hbm_frac_graph": lc["dec_gbs"] / HBM_PEAK_GBS,
            "decode_layer_us_per_step_three_launches": lc["layer_chain_us"],
            "decode_layer_us_per_step_fused": lc["layer_fused_us"],
            "workload": "1 x 1,048,576 tokens, H=96, snapshots every 4096 into 2 slots (automatic plan: two value "
                        "blocks per head), then 128 single-token decode steps (kda_verify n_tok=1, in-place commit), "
                        "one launch per step and as one replayed HIP graph; and a whole decode layer from the "
                        "projections (conv width 4, gated output norm) as kda_prologue + kda_verify + "
                        "kda_gated_rmsnorm per step vs one kda_decode per step, both replayed as graphs",
        }
    if mvs is not None:
        line["state_moves"] = {
            "us": mvs["ms"] * 1e3, "gbs": mvs["gbs"], "hbm_frac": mvs["gbs"] / HBM_PEAK_GBS,
            "workload": "prefix-cache snapshot of 256 requests' working slots (69 layers x 8 heads of 128 x 128 "
                        "fp32 each, 36.2 MB) into fresh slots: one kda_state_move launch, 18.5 GB moved",
        }
    if vf is not None:
        line["verify_fold"] = {
            "us_per_step": (vf["verify_ms"] + vf["fold_ms"]) * 1e3,
            "verify_us": vf["verify_ms"] * 1e3, "fold_us": vf["fold_ms"] * 1e3,
            "verify_hbm_frac": vf["verify_gbs"] / HBM_PEAK_GBS, "fold_hbm_frac": vf["fold_gbs"] / HBM_PEAK_GBS,
            "verify_gbs": vf["verify_gbs"], "fold_gbs": vf["fold_gbs"], "accept_mean": vf["accept_mean"],
            "workload": "256 requests x 69 layers x 8 heads, gamma+1=8 bf16 draft tokens, fp32 committed state, "
                        "ring length 16, accepted lengths geometric mean 2.7 clipped to [1,8]; 69 verify + 1 fold",
            "fused_us_per_step": vf["fused_ms"] * 1e3, "fused_gbs": vf["fused_gbs"],
            "fused_hbm_frac": vf["fused_gbs"] / HBM_PEAK_GBS,
            "fused_workload": "the same step as 69 kda_fold_verify launches (each folds the previous window of "
                              "its layer into the committed state, then verifies the next window from it)",
            "ragged_verify_us_per_step": vf["ragged_ms"] * 1e3, "ragged_gbs": vf["ragged_gbs"],
            "ragged_hbm_frac": vf["ragged_gbs"] / HBM_PEAK_GBS, "ragged_mean_window": vf["ragged_mean_window"],
            "ragged_workload": "the verify of the same step with trimmed windows: request b keeps n_b of its 8 "
                               "draft tokens (uniform on 1..8), packed back to back; 69 kda_verify_ragged launches",
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
