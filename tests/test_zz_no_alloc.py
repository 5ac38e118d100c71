"""kda_chunk_prefill_noalloc (the work list in the library's static device scratch, no workspace
argument) against kda_chunk_prefill with a caller workspace, bit for bit, on two calls in a row on
one stream, the second with a smaller batch (fewer sequences, heads and tokens), and the outputs
against the oracle on sampled units."""
import numpy as np
import pytest
import torch

import synth
import synth.gpu as sg
import linear_attention_recurrence_amd as kda
from kda_ref import TOL, block_err, log, oracle_prefill_unit

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(seed, lens, H, interval, with_s0):
    cu = synth.cu_seqlens(lens)
    T, N = int(cu[-1]), len(lens)
    plan = kda.kda_plan_create(cu, n_heads=H, snap_interval=interval)
    ins = sg.prefill_inputs(seed, T, H, DEV)
    S0 = sg.states(seed, N * H, DEV).view(N, H, 128, 128) if with_s0 else None
    return plan, cu, ins, S0


def _outs(plan, slots):
    T, H, N = plan.total_tokens, plan.n_heads, plan.n_seq
    o = torch.full((T, H, 128), float("nan"), device=DEV)
    st = torch.full((N, H, 128, 128), float("nan"), device=DEV)
    snap = torch.full((N, slots, H, 128, 128), float("nan"), device=DEV) if slots else None
    cnt = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    return o, st, snap, cnt


def _bits(ts):
    return [t.view(torch.int32).clone() for t in ts if t is not None]


def test_noalloc_prefill_matches_workspace_prefill(gpu):
    cases = [  # the second call is smaller in every dimension
        (31, [300, 0, 33, 1000, 64, 129], 6, 64, True),
        (32, [70, 5], 2, 32, False),
    ]
    for seed, lens, H, interval, with_s0 in cases:
        log(f"noalloc prefill: seed {seed}, lengths {lens}, H {H}")
        plan, cu, ins, S0 = _case(seed, lens, H, interval, with_s0)
        a = _outs(plan, 2)
        kda.kda_chunk_prefill_noalloc(plan, *ins, a[1], a[0], state_in=S0, snap=a[2], snap_slots=2, snap_count=a[3])
        b = _outs(plan, 2)
        ws = torch.empty(kda.kda_plan_workspace_bytes(plan), dtype=torch.uint8, device=DEV)
        kda.kda_chunk_prefill(plan, *ins, b[1], b[0], ws, state_in=S0, snap=b[2], snap_slots=2, snap_count=b[3])
        torch.cuda.synchronize()
        for x, y, name in zip(_bits(a), _bits(b), ("o", "state", "snap", "count")):
            assert torch.equal(x, y), f"seed {seed}: {name} differs from kda_chunk_prefill"
        # a stated sample of units against the oracle (normwise per block)
        o_np, st_np = a[0].cpu().numpy(), a[1].cpu().numpy()
        s0_np = S0.cpu().numpy() if S0 is not None else None
        worst = 0.0
        for n in range(len(lens)):
            L = int(lens[n])
            h = n % H
            o_ref, S_ref, _, _ = oracle_prefill_unit(seed, H, int(cu[n]), L, h,
                                                     S0=None if s0_np is None else s0_np[n, h])
            if L:
                worst = max(worst, block_err(o_np[int(cu[n]):int(cu[n + 1]), h], o_ref))
            worst = max(worst, block_err(st_np[n, h], S_ref))
        log(f"noalloc prefill seed {seed}: worst {worst:.2e}")
        assert worst <= TOL
        plan.close()
