"""Benchmark of the KDA hot path on one MI355X.

Headline (``value``): chunked-prefill throughput in tokens*heads/s on the
largest prefill workload, "1 sequence of 1,048,576 tokens, H = 96, K = V =
128, bf16 q/k/v, fp32 gk/beta/state, snapshots every 4096 tokens into 2
ping-pong slots". One step = one kda_chunk_prefill call with the work list
resident (one persistent-kernel launch); each step is timed with HIP events on
the launch stream, after a 1 GiB scratch write (outside the timed region) that
evicts the caches. Beside it, in the same JSON line:

* ``roofline``: HBM roofline of that prefill kernel (algorithmic bytes per
  launch / measured launch time, against 8 TB/s), with the HBM traffic of the
  rocprofv3 counter profile kept under profiles/;
* ``prefill_4x2048_h64``: the dense workload "4 sequences x 2048 tokens,
  H = 64, state_in ~ N(0, 0.1^2)", the same way, plus its output gated RMSNorm
  fused and unfused (``prefill_gated_norm``);
* ``varlen_h96``: "32 sequences, lengths log-uniform in [64, 24576], H = 96,
  snapshots every 2048 into 2 slots", longest-first against input order;
* ``single_head_fp32``: the 64-token fp32 single head (launch-bound);
* ``long_context`` decode: 128 single-token decode steps after the long prefill;
* ``verify_fold``: one speculative step of "256 requests x 69 layers x 8
  heads, gamma + 1 = 8 bf16 draft tokens, ring length 16, accepted lengths
  geometric (mean 2.7, clipped to [1, 8])" = 69 kda_verify launches + one
  kda_replay_fold launch, in us/step (committed states restored from a
  pristine copy outside the timed region before every step); beside it the
  69 verifies replayed as one captured HIP graph (``verify_us_graph``), the
  same step through kda_fold_verify, and the verify with trimmed windows;
* ``prologue``, ``state_moves``: the adjacent steps;
* ``cpu_baseline``: the fp64 oracle (token-by-token) on the host cores this
  process may use, on stated samples of every workload.

Inputs are synthetic, generated on the device by the seeded generator.
"""
from __future__ import annotations

import argparse
import json
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK = 2.5e15  # MI355X dense bf16/fp16 matrix peak, FLOP/s
# algorithmic flops per token*head of the chunked form at the kernel's chunk C = 32, K = V = 128:
# 2 [(3CK + 2CV) / 2 + 3KV] (the five chunk-by-chunk products at their triangular half, the three
# state-shaped products in full)
FLOP_PER_TOKEN_HEAD = 2 * ((3 * 32 * 128 + 2 * 32 * 128) // 2 + 3 * 128 * 128)
METRIC = "KDA prefill tokens*heads/s and verify+fold us/step at 1 GPU; % of roofline"

# HBM bytes per prefill launch measured by rocprofv3 PMC (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000, the
# factors that make a plain 1 GiB copy read 1 GiB and write 1 GiB), per workload; None for a workload
# not measured with the current kernel (set to None whenever the kernel changes until it is measured again)
PREFILL_TRAFFIC_BYTES = {"long_1m_h96": 187_985_215_224, "prefill_4x2048_h64": 994_373_454}
# the same for one launch of each kernel of the speculative step (256 x 69 x 8): kda_verify (chunked),
# kda_replay_fold, kda_fold_verify, kda_verify_ragged
VERIFY_TRAFFIC_BYTES = {"verify": 182_660_442, "fold": 18_941_977_265, "fused": 323_764_716, "ragged": 162_462_854}
FLUSH_BYTES = 1 << 30  # scratch written before every timed prefill rep: evicts the 256 MB Infinity Cache and L2s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--vf-steps", type=int, default=5, help="timed verify+fold steps")
    ap.add_argument("--no-verify-fold", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time only the headline prefill (for profilers)")
    ap.add_argument("--only", choices=["long_1m_h96", "prefill_4x2048_h64", "varlen_h96", "verify_fold"],
                    help="time only this workload (for profilers); no JSON headline unless it is long_1m_h96")
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


def workload_bytes(lens, H, with_state_in, snap_interval):
    """prefill_bytes for a batch of lengths, plus 64 KiB per snapshot written."""
    tot = int(sum(int(x) for x in lens))
    snaps = sum(int(x) // snap_interval for x in lens) if snap_interval else 0
    return tot * H * 1796 + len(lens) * H * 65536 * (2 if with_state_in else 1) + snaps * H * 65536


def settle(step, torch, seconds=0.25):
    """Run the step untimed until `seconds` of wall time have passed: the GPU's clocks ramp up
    over the first ~100 launches of a short kernel, and the timed region should see the steady
    state. This precedes the W warm-up steps and is never part of the timed region."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()


def time_reps(torch, step, reps, flush):
    """Time `reps` calls of step(), each on its own with HIP events on the launch stream (the current
    stream, which the binding launches on). Before each, outside the events, the 1 GiB scratch `flush`
    is written on the same stream; the start event is recorded while that write still runs, so the
    stream never idles between the event and the launch. Returns the per-call times in ms."""
    stream = torch.cuda.current_stream()
    out = []
    for r in range(reps):
        torch.cuda.synchronize()
        flush.fill_(float(r & 7))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def summary(times):
    ts = sorted(times)
    return dict(mean_ms=sum(ts) / len(ts), median_ms=ts[len(ts) // 2], min_ms=ts[0], reps=len(ts))


def bench_prefill_workload(name, orders, reps, warmup, torch, kda, sg, synth, flush, v_blocks=1, short=False):
    """One prefill workload of synth.PREFILL_CONFIGS on the device: every order in `orders` (a plan per
    order, the work list resident), `warmup` untimed calls then `reps` timed ones each, a cache flush
    before every timed call. Returns per order the time summary, plus the workload's sizes."""
    dev = "cuda:0"
    c = synth.PREFILL_CONFIGS[name]
    seed, H = c["seed"], c["H"]
    lens = synth.prefill_lengths(name)
    cu = synth.cu_seqlens(lens)
    T, N = int(cu[-1]), len(lens)
    ins = sg.prefill_inputs(seed, T, H, dev)
    S0 = sg.states(seed, N * H, dev).view(N, H, 128, 128) if c["state_in"] == "normal" else None
    o = torch.empty((T, H, 128), device=dev)
    st = torch.empty((N, H, 128, 128), device=dev)
    slots = c["snap_slots"]
    snap = torch.empty((N, slots, H, 128, 128), device=dev) if slots else None
    cnt = torch.empty((N,), dtype=torch.int32, device=dev)
    res = {}
    for order in orders:
        plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=c["snap_interval"], order=order, v_blocks=v_blocks)
        ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=dev)
        kda.kda_plan_upload(plan, ws)

        def step():
            kda.kda_chunk_prefill(plan, *ins, st, o, ws, state_in=S0, snap=snap, snap_slots=slots, snap_count=cnt,
                                  flags=kda.KDA_PREFILL_PLAN_RESIDENT)

        if short:
            settle(step, torch)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        r = summary(time_reps(torch, step, reps, flush))
        r["items"] = kda.kda_plan_num_items(plan)
        r["v_blocks"] = kda.kda_plan_v_blocks(plan)
        res[order] = r
        plan.close()
    byts = workload_bytes(lens, H, S0 is not None, c["snap_interval"] if slots else 0)
    out = dict(res=res, bytes=byts, tokens_heads=T * H, T=T, N=N, H=H, lens=lens, st=st)
    del ins, o, snap, S0
    return out


def bench_single_head(torch, kda, sg, synth, flush):
    """The 64-token fp32 single head (state zero): kda_verify on the fp32 inputs (n_tok = 64, no ring,
    commit after 64) and kda_chunk_prefill on bf16-rounded copies of q, k, v. Launch-bound: us per call."""
    dev = "cuda:0"
    c = synth.PREFILL_CONFIGS["single_64"]
    seed, T = c["seed"], c["lengths"][0]
    q, k, v, gk, beta = sg.prefill_inputs(seed, T, 1, dev, qkv_dtype=torch.float32)
    pool = torch.zeros((1, 1, 1, 128, 128), device=dev)
    commit = torch.empty_like(pool)
    slot = torch.zeros(1, dtype=torch.int32, device=dev)
    clen = torch.full((1,), T, dtype=torch.int32, device=dev)
    o = torch.empty((T, 1, 128), device=dev)

    def verify():
        kda.kda_verify(q, k, v, gk, beta, pool, slot, o, layer=0, n_tok=T, commit_len=clen, commit_pool=commit)

    qb, kb, vb = (x.to(torch.bfloat16) for x in (q, k, v))
    plan = kda.kda_plan_create(synth.cu_seqlens([T]), n_heads=1)
    ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=dev)
    kda.kda_plan_upload(plan, ws)
    st = torch.empty((1, 1, 128, 128), device=dev)

    def prefill():
        kda.kda_chunk_prefill(plan, qb, kb, vb, gk, beta, st, o, ws, flags=kda.KDA_PREFILL_PLAN_RESIDENT)

    out = {}
    for name, fn in (("verify_fp32", verify), ("prefill_bf16", prefill)):
        settle(fn, torch, 0.1)
        out[name] = summary(time_reps(torch, fn, 20, flush))
    plan.close()
    return out


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


def bench_decode(st, torch, kda, sg, synth):
    """128 single-token decode steps of the long-context workload from its prefill's final state `st`
    ([1, 96, 128, 128]): kda_verify (n_tok = 1, commit in place), launched one by one and as one replayed
    HIP graph; then a whole decode layer from the projections as three launches per step and as one
    kda_decode per step, both replayed as graphs."""
    dev = "cuda:0"
    c = synth.PREFILL_CONFIGS["long_1m_h96"]
    seed, H = c["seed"], c["H"]
    stream = torch.cuda.current_stream()
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
    return dict(eager_us=eager_us, graph_us=graph_us, dec_gbs=dec_bytes / (graph_us * 1e-6) / 1e9,
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

    # The 69 verifies again, captured once as a HIP graph and replayed, as a serving loop launches a
    # step's kernels: the same launches with the host's per-call work and most of the gaps between
    # kernels taken out. They only read the committed pool and rewrite the ring with the same bits.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(Lyr):
            q, k, v, gk, beta = ins[l]
            kda.kda_verify(q, k, v, gk, beta, pool, slot_idx, o, layer=l, n_tok=T, ring=ring, ring_start=ring_start)
    graph.replay()
    torch.cuda.synchronize()
    gtimes = []
    for _ in range(args.vf_steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        graph.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        gtimes.append(ev[0].elapsed_time(ev[1]))
    ver_graph = sum(gtimes) / len(gtimes)
    del graph

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
    res = dict(verify_ms=ver, fold_ms=fol, accept_mean=acc_mean, verify_graph_ms=ver_graph,
               verify_graph_gbs=v_bytes / (ver_graph * 1e-3) / 1e9,
               verify_gbs=v_bytes / (ver * 1e-3) / 1e9, fold_gbs=f_bytes / (fol * 1e-3) / 1e9,
               verify_bytes=v_bytes, fold_bytes=f_bytes, fused_ms=fus, fused_bytes=fv_bytes,
               fused_gbs=fv_bytes / (fus * 1e-3) / 1e9, ragged_ms=rag, ragged_bytes=r_bytes,
               ragged_gbs=r_bytes / (rag * 1e-3) / 1e9, ragged_mean_window=float(win.mean()), layers=Lyr)
    del pool, pristine, ring, ins_r, o, o_r
    return res


def measure_peaks(torch, kda, reps=5):
    """The rates this GPU attains on the simplest work, through the library's measurement probes in the
    same run: a streaming copy of 1 GiB (2 GiB moved), a streaming read of the same 1 GiB, and a loop of
    independent bf16 16x16x32 MFMAs over two workgroups per CU. Median of `reps` launches after one
    untimed launch each, timed with HIP events on the launch stream."""
    dev = "cuda:0"
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(4096 * 256, device=dev)

    def med(fn):
        fn()
        ts = []
        for _ in range(reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        return statistics.median(ts)

    t_copy = med(lambda: kda.kda_probe_copy(dst, src))
    t_read = med(lambda: kda.kda_probe_read(src, sink))
    flop = [0]
    iters = 20000

    def mf():
        flop[0] = kda.kda_probe_mfma(iters, sink)

    t_mfma = med(mf)
    del src, dst, sink
    torch.cuda.empty_cache()
    return {"hbm_copy_gbs": 2 * nbytes / t_copy / 1e9, "hbm_read_gbs": nbytes / t_read / 1e9,
            "mfma_bf16_tflops": flop[0] / t_mfma / 1e12,
            "probes": "kda_probe_copy of 1 GiB (2 GiB moved) and kda_probe_read of 1 GiB, non-temporal float4 "
                      "streams; kda_probe_mfma with "
                      f"{iters} rounds of 8 independent 16x16x32 bf16 MFMAs per wave; medians of {reps}"}


def host_cores():
    """(threads to use, nproc, CPUs this process may run on, CPU model). The oracle runs one unit per task
    on the CPUs this process may use, capped by OMP_NUM_THREADS when the environment sets it (the share of
    host cores a one-GPU job is given)."""
    nproc = os.cpu_count() or 1
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = nproc
    threads = aff
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        threads = min(threads, int(env))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, nproc, aff, model


def cpu_baseline(synth, oracle):
    """The fp64 oracle, as it is (token-by-token, one (sequence, head) or (request, layer, head) unit per
    task), on stated samples of every workload. Input generation is not timed. A sample keeps the
    workload's shapes and distributions, so its rate is the workload's rate."""
    import numpy as np

    threads, nproc, aff, model = host_cores()

    def timed_units(units, prep, run, batch=None):
        # inputs of `batch` units at a time are prepared (untimed), then run (timed), so that the fp64
        # inputs of a large sample never sit in host memory all at once
        batch = batch or len(units)
        dt = 0.0
        for i in range(0, len(units), batch):
            part = units[i:i + batch]
            data = dict(zip(part, oracle.run_parallel(prep, part, threads=threads)))
            t0 = time.perf_counter()
            oracle.run_parallel(lambda u: run(data[u]), part, threads=threads)
            dt += time.perf_counter() - t0
            del data
        return dt

    def prefill_prep(name, t0_fn, L_fn, with_s0):
        c = synth.PREFILL_CONFIGS[name]

        def prep(u):
            n, h = u
            q, k, v, gk, beta = synth.prefill_rows(c["seed"], c["H"], t0_fn(n), L_fn(n), h=h)
            S0 = synth.state_rows(c["seed"], n * c["H"] + h, 1)[0] if with_s0 else None
            return tuple(oracle.f64(x) for x in (q, k, v, gk, beta)) + (S0,)
        return prep

    def prefill_run(d):
        q, k, v, gk, beta, S0 = d
        oracle.recurrent(q, k, v, gk, beta, S0)

    out = {}
    # single head, 64 tokens, fp32: the whole workload
    c0 = synth.PREFILL_CONFIGS["single_64"]
    q, k, v, gk, beta = synth.prefill_rows(c0["seed"], 1, 0, 64, h=0, qkv_dtype=synth.F32)
    args0 = tuple(oracle.f64(x) for x in (q, k, v, gk, beta))
    t0 = time.perf_counter()
    for _ in range(200):
        oracle.recurrent(*args0)
    dt = (time.perf_counter() - t0) / 200
    out["single_head_fp32"] = dict(value=64 / dt, unit="tokens*heads/s", sample="the whole workload (1 head x 64 "
                                   f"tokens), mean of 200 runs: {dt * 1e6:.0f} us each")
    # 4 x 2048, H64: every unit
    L1 = 2048
    units = [(n, h) for n in range(4) for h in range(64)]
    dt = timed_units(units, prefill_prep("prefill_4x2048_h64", lambda n: n * L1, lambda n: L1, True), prefill_run)
    out["prefill_4x2048_h64"] = dict(value=len(units) * L1 / dt, unit="tokens*heads/s",
                                     sample=f"the whole workload: 256 (sequence, head) units x 2048 tokens, {dt:.2f} s")
    # varlen H96: every sequence, 8 heads (0, 12, .., 84)
    lens = synth.prefill_lengths("varlen_h96")
    cu = synth.cu_seqlens(lens)
    heads = list(range(0, 96, 12))
    units = [(n, h) for n in range(len(lens)) for h in heads]
    dt = timed_units(units, prefill_prep("varlen_h96", lambda n: int(cu[n]), lambda n: int(lens[n]), False),
                     prefill_run)
    th = int(sum(lens)) * len(heads)
    out["varlen_h96"] = dict(value=th / dt, unit="tokens*heads/s",
                             sample=f"all 32 sequences ({int(sum(lens))} tokens) x heads {heads} (fp64, no "
                                    f"snapshot copies), {dt:.2f} s")
    # long context: all 96 heads over the first 262,144 of the 1,048,576 tokens, 16 heads at a time
    L4 = 262144
    units = [(0, h) for h in range(96)]
    dt = timed_units(units, prefill_prep("long_1m_h96", lambda n: 0, lambda n: L4, False), prefill_run, batch=16)
    out["long_1m_h96"] = dict(value=L4 * len(units) / dt, unit="tokens*heads/s",
                              sample=f"all 96 heads over tokens 0..{L4 - 1} of the 1,048,576 (the per-token cost "
                                     f"does not depend on the position), inputs prepared 16 heads at a time, "
                                     f"{dt:.2f} s timed")
    # speculative step: layer 0 of the 256 x 69 x 8 step (2,048 units): verify 8 tokens (ring recorded),
    # then fold the accepted prefix; scaled by 69 layers to ms/step
    vc = synth.VERIFY_CONFIG
    acc = synth.geometric_accept(vc["seed"], vc["B"])
    units = [(b, h) for b in range(vc["B"]) for h in range(vc["H"])]

    def vprep(u):
        b, h = u
        q, k, v, gk, beta = synth.prefill_rows(vc["seed"], vc["H"], b * vc["T"], vc["T"], h=h, sub=0)
        S0 = synth.state_rows(vc["seed"], (b * vc["L"] + 0) * vc["H"] + h, 1)[0]
        return tuple(oracle.f64(x) for x in (q, k, v, gk, beta)) + (S0, int(acc[b]))

    def vrun(d):
        q, k, v, gk, beta, S0, n = d
        _, _, ring = oracle.verify(q, k, v, gk, beta, S0)
        S = np.array(S0, dtype=np.float64)
        oracle.fold(n, ring["k"], ring["v"], ring["gk"], ring["beta"], S)

    dt = timed_units(units, vprep, vrun)
    out["verify_fold_256x69x8"] = dict(value=dt * vc["L"] * 1e3, unit="ms/step",
                                       sample=f"layer 0 of the step (256 requests x 8 heads: verify 8 tokens, then "
                                              f"fold the accepted prefix), {dt:.2f} s, x 69 layers")
    head = out["long_1m_h96"]
    return dict(value=head["value"], unit="tokens*heads/s", cores=threads, kind="oracle",
                sample="long-context prefill: " + head["sample"], nproc=nproc, cpus_allowed=aff, cpu_model=model,
                workloads=out)


def prefill_leg(r, order, synth_name, traffic=None):
    """JSON fields of one timed prefill workload in one order: time, throughput, HBM and MFMA fractions."""
    t = r["res"][order]
    ms = t["mean_ms"]
    gbs = r["bytes"] / (ms * 1e-3) / 1e9
    flops = r["tokens_heads"] * FLOP_PER_TOKEN_HEAD
    return {"ms": ms, "median_ms": t["median_ms"], "min_ms": t["min_ms"], "reps": t["reps"],
            "tokens_heads_per_s": r["tokens_heads"] / (ms * 1e-3), "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "mfma_frac": flops / (ms * 1e-3) / MFMA_BF16_PEAK, "algorithmic_bytes": r["bytes"],
            "items": t["items"], "v_blocks": t["v_blocks"], "traffic": traffic}


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
    only = args.only
    if args.verify_fold_only:
        only = "verify_fold"
    if args.prefill_only:
        only = "long_1m_h96"
    want = (lambda name: only is None or only == name)
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    LPT, FIFO = kda.KDA_PLAN_LPT, kda.KDA_PLAN_FIFO
    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}

    head = None
    if want("long_1m_h96"):
        log("long context: 1M x 96 prefill (the headline)")
        try:
            lc = bench_prefill_workload("long_1m_h96", [LPT], args.steps, args.warmup, torch, kda, sg, synth, flush,
                                        v_blocks=0)
            head = prefill_leg(lc, LPT, "long_1m_h96", PREFILL_TRAFFIC_BYTES["long_1m_h96"])
            log(f"long context: {head['ms']:.2f} ms/launch, {head['gbs']:.0f} GB/s")
            st = lc["st"]
            del lc
            torch.cuda.empty_cache()
            if only is None:
                log("long context: 128 decode steps")
                dec = bench_decode(st, torch, kda, sg, synth)
                head["decode"] = {
                    "us_per_step_eager": dec["eager_us"], "us_per_step_graph": dec["graph_us"],
                    "gbs_graph": dec["dec_gbs"], "hbm_frac_graph": dec["dec_gbs"] / HBM_PEAK_GBS,
                    "layer_us_per_step_three_launches": dec["layer_chain_us"],
                    "layer_us_per_step_fused": dec["layer_fused_us"],
                    "workload": "128 single-token decode steps from the long prefill's final state (kda_verify "
                                "n_tok=1, in-place commit, 96 heads), one launch per step and as one replayed HIP "
                                "graph; and a whole decode layer from the projections (conv width 4, gated output "
                                "norm) as kda_prologue + kda_verify + kda_gated_rmsnorm per step vs one kda_decode "
                                "per step, both replayed as graphs"}
            del st
        except torch.cuda.OutOfMemoryError as e:  # the line must still be printed
            log(f"long context skipped: {e}")
        torch.cuda.empty_cache()

    dense = None
    if want("prefill_4x2048_h64"):
        log("prefill 4 x 2048, H64")
        r = bench_prefill_workload("prefill_4x2048_h64", [LPT], args.steps, args.warmup, torch, kda, sg, synth, flush,
                                   short=True)
        dense = prefill_leg(r, LPT, "prefill_4x2048_h64", PREFILL_TRAFFIC_BYTES["prefill_4x2048_h64"])
        log(f"prefill 4 x 2048: {dense['ms'] * 1e3:.1f} us/launch, {dense['gbs']:.0f} GB/s")
        del r
        torch.cuda.empty_cache()
    varlen = None
    if want("varlen_h96"):
        log("varlen H96 prefill: longest-first and input order")
        r = bench_prefill_workload("varlen_h96", [LPT, FIFO], 10, 2, torch, kda, sg, synth, flush, short=True)
        varlen = {"lpt": prefill_leg(r, LPT, "varlen_h96"), "fifo": prefill_leg(r, FIFO, "varlen_h96"),
                  "total_tokens": int(sum(r["lens"])), "n_seq": r["N"], "heads": r["H"]}
        varlen["lpt_speedup"] = varlen["fifo"]["ms"] / varlen["lpt"]["ms"]
        log(f"varlen: LPT {varlen['lpt']['ms']:.3f} ms, FIFO {varlen['fifo']['ms']:.3f} ms")
        del r
        torch.cuda.empty_cache()
    single = bench_single_head(torch, kda, sg, synth, flush) if only is None else None
    pg = pro = mvs = None
    if only is None:
        log("prefill with the output gated RMSNorm: fused and unfused")
        pg = bench_prefill_gated(args, torch, kda, sg, synth)
        log("prologue")
        pro = bench_prologue(args, torch, kda, sg, synth)
        log("state moves")
        mvs = bench_state_moves(args, torch, kda, sg, synth)
    del flush
    torch.cuda.empty_cache()
    vf = None
    if want("verify_fold") and not args.no_verify_fold:
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
    peaks = None
    if only is None:
        log("attained peaks: copy, read and MFMA probes")
        peaks = measure_peaks(torch, kda)
        log(f"attained peaks: copy {peaks['hbm_copy_gbs']:.0f} GB/s, read {peaks['hbm_read_gbs']:.0f} GB/s, "
            f"bf16 MFMA {peaks['mfma_bf16_tflops']:.0f} TFLOP/s")
    cpu = None
    if only is None and not args.no_cpu_baseline:
        import oracle

        log("cpu baseline: fp64 oracle on host cores")
        cpu = cpu_baseline(synth, oracle)

    if head is not None:
        line.update({
            "value": head["tokens_heads_per_s"], "unit": "tokens*heads/s", "ms_per_step": head["ms"],
            "config": {"workload": "long-context chunked prefill: 1 sequence x 1,048,576 tokens, H=96, K=V=128, "
                                   "bf16 q/k/v, fp32 gk/beta/state, state_in zero, snapshots every 4096 tokens into "
                                   "2 ping-pong slots, chunk 32, one persistent launch (two value blocks per head)",
                       "n_seq": 1, "seq_len": 1048576, "heads": 96, "head_dim": 128},
            "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": head["hbm_frac"], "traffic": head["traffic"], "kernel": "kda::prefill_kernel<false>",
                         "algorithmic_bytes_per_launch": head["algorithmic_bytes"], "mfma_frac": head["mfma_frac"],
                         "median_ms": head["median_ms"], "min_ms": head["min_ms"]},
        })
        if peaks is not None:
            line["roofline"]["frac_of_attained_copy"] = head["gbs"] / peaks["hbm_copy_gbs"]
            line["roofline"]["frac_of_attained_read"] = head["gbs"] / peaks["hbm_read_gbs"]
        line["long_context"] = head
    elif dense is not None:
        line.update({
            "value": dense["tokens_heads_per_s"], "unit": "tokens*heads/s", "ms_per_step": dense["ms"],
            "config": {"workload": "chunked prefill: 4 sequences x 2048 tokens, H=64 (the long-context workload "
                                   "did not run)", "n_seq": 4, "seq_len": 2048, "heads": 64, "head_dim": 128},
            "roofline": {"bound": "hbm", "achieved": dense["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dense["hbm_frac"], "traffic": dense["traffic"], "kernel": "kda::prefill_kernel<false>",
                         "algorithmic_bytes_per_launch": dense["algorithmic_bytes"]},
        })
    line["attained_peaks"] = peaks
    line["cpu_baseline"] = cpu
    if dense is not None:
        dense["workload"] = ("4 sequences x 2048 tokens, H=64, bf16 q/k/v, fp32 gk/beta/state, state_in N(0,0.1^2), "
                             "no snapshots (one value block per head)")
        line["prefill_4x2048_h64"] = dense
    if varlen is not None:
        varlen["workload"] = ("32 sequences, lengths log-uniform in [64, 24576] (seed 2), H=96, state_in zero, "
                              "snapshots every 2048 tokens into 2 slots; the persistent kernel pulling (sequence, "
                              "head) items longest-first (lpt) vs in input order (fifo)")
        line["varlen_h96"] = varlen
    if single is not None:
        line["single_head_fp32"] = {
            "verify_fp32_us": single["verify_fp32"]["median_ms"] * 1e3,
            "prefill_bf16_us": single["prefill_bf16"]["median_ms"] * 1e3,
            "workload": "1 head x 64 tokens, state zero: kda_verify on fp32 inputs (n_tok 64, commit after 64) and "
                        "kda_chunk_prefill on bf16-rounded q/k/v (launch-bound; medians of 20 calls)"}
    if pg is not None:
        line["prefill_gated_norm"] = {
            "fused_us": pg["fused_ms"] * 1e3, "unfused_us": pg["unfused_ms"] * 1e3,
            "fused_tokens_heads_per_s": pg["tokens_heads"] / (pg["fused_ms"] * 1e-3),
            "fused_gbs": pg["fused_bytes"] / (pg["fused_ms"] * 1e-3) / 1e9,
            "fused_hbm_frac": pg["fused_bytes"] / (pg["fused_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "workload": "the 4 x 2048, H64 prefill followed by the output gated RMSNorm (gate N(0,1) bf16, weights "
                        "1 + 0.1 N(0,1), eps 1e-6, bf16 y): kda_chunk_prefill_gated vs kda_chunk_prefill + "
                        "kda_gated_rmsnorm (back-to-back launches)",
        }
    if pro is not None:
        line["prologue"] = {
            "us": pro["ms"] * 1e3, "gbs": pro["gbs"], "hbm_frac": pro["gbs"] / HBM_PEAK_GBS,
            "workload": "kda_prologue over the 4 x 2048, H64 batch: conv width 4 with the state carried in and out, "
                        "SiLU, q/k L2 norm, beta sigmoid, gk = -softplus (2,568 B per token*head)",
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
            "step_hbm_frac": (vf["verify_bytes"] + vf["fold_bytes"]) / ((vf["verify_ms"] + vf["fold_ms"]) * 1e-3)
                             / 1e9 / HBM_PEAK_GBS,
            "verify_gbs": vf["verify_gbs"], "fold_gbs": vf["fold_gbs"], "accept_mean": vf["accept_mean"],
            "verify_us_graph": vf["verify_graph_ms"] * 1e3,
            "verify_hbm_frac_graph": vf["verify_graph_gbs"] / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": {"verify": vf["verify_bytes"] // vf["layers"], "fold": vf["fold_bytes"],
                                             "fused": vf["fused_bytes"] // vf["layers"],
                                             "ragged": vf["ragged_bytes"] // vf["layers"]},
            "traffic_per_launch": VERIFY_TRAFFIC_BYTES,
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
