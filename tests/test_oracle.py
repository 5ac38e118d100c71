"""Pins of the fp64 oracle (CPU only).

Nothing here compares the oracle with itself under another name: every check
is against a closed form, an invariant of the recurrence, the textbook
full-matrix form of the delta rule, an independently derived chunked algebra,
or the sizes the pages print (tests/golden/sizes.json). Each is chosen so a
plausible slip (a dropped decay, the error taken against the undecayed state,
readout before the update, a sign, a transposed state) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_inputs(rng, L, K, V, unit_k=True):
    q = rng.standard_normal((L, K))
    k = rng.standard_normal((L, K))
    if unit_k:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((L, V))
    gk = -np.log1p(np.exp(rng.standard_normal((L, K))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    return q, k, v, gk, beta


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# I1: beta = 0 and gk = 0 leave the state unchanged; o_t = scale * S0^T q_t
def test_identity_step_leaves_state():
    rng = np.random.default_rng(1)
    L, K, V = 7, 6, 5
    q, k, v, gk, beta = rand_inputs(rng, L, K, V)
    S0 = rng.standard_normal((K, V))
    o, S, _, _ = oracle.recurrent(q, k, v, np.zeros_like(gk), np.zeros(L), S0, scale=0.37)
    assert np.array_equal(S, S0)
    assert rel(o, 0.37 * q @ S0) < 1e-14


# decay is applied before the delta update: with beta = 1 and k = e_r, row r
# of the new state is exactly v and every other row is a[c] * S0[c]
def test_decay_then_delta_order():
    rng = np.random.default_rng(2)
    K, V, r = 5, 4, 3
    S0 = rng.standard_normal((K, V))
    k = np.zeros((1, K))
    k[0, r] = 1.0
    v = rng.standard_normal((1, V))
    gk = -rng.uniform(0.1, 2.0, (1, K))
    q = rng.standard_normal((1, K))
    _, S, _, _ = oracle.recurrent(q, k, v, gk, np.ones(1), S0)
    a = np.exp(gk[0])
    want = a[:, None] * S0
    want[r] = v[0]
    assert rel(S, want) < 1e-15


# the readout uses the updated state: from S0 = 0 one token gives
# o = scale * beta * (q . k) * v   (it would be 0 if read before the update)
def test_readout_after_update():
    rng = np.random.default_rng(3)
    K, V = 8, 6
    q, k, v, gk, beta = rand_inputs(rng, 1, K, V)
    o, _, _, _ = oracle.recurrent(q, k, v, gk, beta, None, scale=1.7)
    want = 1.7 * beta[0] * float(q[0] @ k[0]) * v[0]
    assert rel(o[0], want) < 1e-14


# I5: with beta = 1 and ||k|| = 1 exactly, the new state maps k to v
def test_delta_rule_writes_value_at_key():
    rng = np.random.default_rng(4)
    K, V = 8, 5
    S0 = rng.standard_normal((K, V))
    for kv in ([0.6, 0.8], [0.5, -0.5, 0.5, -0.5]):
        k = np.zeros((1, K))
        k[0, : len(kv)] = kv  # norm exactly 1 in binary floating point
        v = rng.standard_normal((1, V))
        gk = -rng.uniform(0.0, 1.5, (1, K))
        _, S, _, _ = oracle.recurrent(rng.standard_normal((1, K)), k, v, gk, np.ones(1), S0)
        assert np.max(np.abs(S.T @ k[0] - v[0])) < 1e-14


# I6: beta = 0 everywhere leaves only the decay: S_T = diag(exp(sum_t gk_t)) S0
def test_pure_decay():
    rng = np.random.default_rng(5)
    L, K, V = 23, 7, 3
    q, k, v, gk, _ = rand_inputs(rng, L, K, V)
    S0 = rng.standard_normal((K, V))
    _, S, _, _ = oracle.recurrent(q, k, v, gk, np.zeros(L), S0)
    assert rel(S, np.exp(gk.sum(0))[:, None] * S0) < 1e-13


# I7: with (q, k, gk, beta) fixed, (S0, v) -> (S_T, o) is linear
def test_linearity_in_state_and_values():
    rng = np.random.default_rng(6)
    L, K, V = 11, 6, 4
    q, k, v1, gk, beta = rand_inputs(rng, L, K, V)
    v2 = rng.standard_normal((L, V))
    S1, S2 = rng.standard_normal((K, V)), rng.standard_normal((K, V))
    x, y = 0.7, -1.3
    o1, T1, _, _ = oracle.recurrent(q, k, v1, gk, beta, S1)
    o2, T2, _, _ = oracle.recurrent(q, k, v2, gk, beta, S2)
    o3, T3, _, _ = oracle.recurrent(q, k, x * v1 + y * v2, gk, beta, x * S1 + y * S2)
    assert rel(o3, x * o1 + y * o2) < 1e-13
    assert rel(T3, x * T1 + y * T2) < 1e-13


# I8: gk = -inf (decay factor 0) resets the state to beta_t k_t v_t^T each token
def test_full_reset():
    rng = np.random.default_rng(7)
    L, K, V = 4, 5, 3
    q, k, v, _, beta = rand_inputs(rng, L, K, V)
    S0 = rng.standard_normal((K, V))
    o, S, _, _ = oracle.recurrent(q, k, v, np.full((L, K), -np.inf), beta, S0)
    assert rel(S, beta[-1] * np.outer(k[-1], v[-1])) < 1e-15
    for t in range(L):
        assert rel(o[t], beta[t] * float(q[t] @ k[t]) * v[t]) < 1e-14


# I9: textbook full-matrix delta rule S <- (I - beta k k^T) diag(a) S + beta k v^T,
# on tiny K, V (K != V catches a transposed state)
@pytest.mark.parametrize("K,V", [(1, 1), (2, 4), (4, 2), (8, 8), (3, 7)])
def test_brute_force_matrix_form(K, V):
    rng = np.random.default_rng(100 + 10 * K + V)
    L = 9
    q, k, v, gk, beta = rand_inputs(rng, L, K, V, unit_k=False)
    S0 = rng.standard_normal((K, V))
    o, S, _, _ = oracle.recurrent(q, k, v, gk, beta, S0, scale=0.9)
    M = S0.copy()
    for t in range(L):
        P = np.eye(K) - beta[t] * np.outer(k[t], k[t])
        M = P @ np.diag(np.exp(gk[t])) @ M + beta[t] * np.outer(k[t], v[t])
        assert np.max(np.abs(o[t] - 0.9 * M.T @ q[t])) <= 1e-13 * max(1.0, np.max(np.abs(M)))
    assert np.max(np.abs(S - M)) <= 1e-13 * max(1.0, np.max(np.abs(M)))


# I2: the chunked (WY/UT) algebra reaches the token loop's result
@pytest.mark.parametrize("C", [1, 2, 8, 32, 64])
@pytest.mark.parametrize("L", [1, 31, 33, 100])
def test_chunked_equals_token_loop(C, L):
    rng = np.random.default_rng(1000 + C * 7 + L)
    K, V = 16, 8
    q, k, v, gk, beta = rand_inputs(rng, L, K, V)
    S0 = 0.1 * rng.standard_normal((K, V))
    o1, S1, _, _ = oracle.recurrent(q, k, v, gk, beta, S0, scale=0.8)
    o2, S2 = oracle.chunked(q, k, v, gk, beta, S0, scale=0.8, chunk=C)
    assert rel(o2, o1) < 1e-12
    assert rel(S2, S1) < 1e-12


# I3: verify + fold of the first n steps == n recurrent steps, bitwise; verify
# never writes the committed state; its commit equals the recurrent state
@pytest.mark.parametrize("n", range(0, 9))
def test_verify_fold_equals_recurrence(n):
    rng = np.random.default_rng(200 + n)
    T, K, V = 8, 12, 10
    q, k, v, gk, beta = rand_inputs(rng, T, K, V)
    S0 = 0.1 * rng.standard_normal((K, V))
    S0_keep = S0.copy()
    o_v, S_commit, ring = oracle.verify(q, k, v, gk, beta, S0, scale=1.0, commit_len=n)
    assert np.array_equal(S0, S0_keep)
    o_r, S_n, _, _ = oracle.recurrent(q[:n], k[:n], v[:n], gk[:n], beta[:n], S0)
    o_full, _, _, _ = oracle.recurrent(q, k, v, gk, beta, S0)
    assert np.array_equal(o_v, o_full)
    if n > 0:
        assert np.array_equal(S_commit, S_n)
    for key, src in (("k", k), ("v", v), ("gk", gk), ("beta", beta)):
        assert np.array_equal(ring[key], src)
    S = S0.copy()
    oracle.fold(n, ring["k"], ring["v"], ring["gk"], ring["beta"], S)
    assert np.array_equal(S, S_n)
    # rejected steps are never replayed: garbage beyond n changes nothing
    ring2 = {key: val.copy() for key, val in ring.items()}
    for key in ring2:
        ring2[key][n:] = np.nan
    S2 = S0.copy()
    oracle.fold(n, ring2["k"], ring2["v"], ring2["gk"], ring2["beta"], S2)
    assert np.array_equal(S2, S_n)


# I4: a restored snapshot continues identically (bitwise in the oracle),
# snapshot slots follow the ping-pong rule, and the last snapshot equals the
# final state when the length is a multiple of the interval
def test_snapshot_restore_and_slots():
    rng = np.random.default_rng(300)
    L, K, V, iv, slots = 96, 8, 6, 16, 2
    q, k, v, gk, beta = rand_inputs(rng, L, K, V)
    S0 = rng.standard_normal((K, V))
    o, S, snaps, cnt = oracle.recurrent(q, k, v, gk, beta, S0, snap_interval=iv, snap_slots=slots)
    assert cnt == L // iv
    # the last two snapshots are positions 80 (m=5 -> slot 0) and 96 (m=6 -> slot 1)
    _, S80, _, _ = oracle.recurrent(q[:80], k[:80], v[:80], gk[:80], beta[:80], S0)
    assert np.array_equal(snaps[0], S80)
    assert np.array_equal(snaps[1], S)  # L % iv == 0: last snapshot == final state
    # resume from the snapshot at 80 and feed the rest with pos0 = 80
    o2, S2, snaps2, cnt2 = oracle.recurrent(q[80:], k[80:], v[80:], gk[80:], beta[80:], S80, pos0=80,
                                            snap_interval=iv, snap_slots=slots)
    assert np.array_equal(S2, S)
    assert np.array_equal(o2, o[80:])
    assert cnt2 == 1 and np.array_equal(snaps2[1], S)


def test_length_zero_is_identity():
    S0 = np.arange(12.0).reshape(3, 4)
    e = np.zeros((0, 3))
    o, S, _, _ = oracle.recurrent(e, e, np.zeros((0, 4)), e, np.zeros(0), S0)
    assert o.shape == (0, 4) and np.array_equal(S, S0)


# I10: the pages' closed-form sizes, from this build's layout (fp32 state,
# K = V = 128, ring entry = bf16 k and v, fp32 gk, fp32 beta)
def test_sizes_match_pages():
    g = json.load(open(os.path.join(HERE, "golden", "sizes.json")))
    d = g["head_dim"]
    state = d * d * 4
    entry = d * 2 + d * 2 + d * 4 + 4
    assert state == g["state_bytes_per_unit_kib"] * 1024
    assert abs(entry / 1024 - g["raw_input_bytes_approx_kib"]) < 0.05  # 1,028 B, "about 1 KB"
    gamma = 7
    assert (gamma + 1) * state == g["draft_window_before_kib"] * 1024
    ring16 = 16 * entry
    assert abs(ring16 / 1024 - g["draft_window_after_kib"]) < 0.1  # 16,448 B, "16 KB"
    assert abs((gamma + 1) * state / ring16 - g["draft_window_ratio_approx"]) < 0.2
    per_req_tp8 = g["kda_layers"] * (g["heads_per_layer"] // g["tp"]) * state
    assert abs(per_req_tp8 / 1e6 - g["state_per_request_tp8_mb_approx"]) < 1.0
    per_step_tp1 = g["kda_layers"] * g["heads_per_layer"] * state
    assert abs(per_step_tp1 / 1e9 - g["state_per_step_tp1_gb_approx"]) < 0.01
    for ex in g["ring_rule_examples"]:
        m = 2 * (ex["gamma"] + 1)
        assert m == ex["min_len"]
        assert 1 << math.ceil(math.log2(m)) == ex["len"]


# ---------------------------------------------------------------- output gated RMSNorm
# The pages name the operation (a gated RMSNorm on the KDA output) but not its formula; these pin the
# oracle's reading of it: divide each row by its root mean square (eps inside the root), scale by a
# per-channel weight, multiply by the logistic sigmoid of the gate.

def test_gated_rmsnorm_unit_rms_with_open_gate():
    """w = 1, eps = 0 and a gate far in saturation: every row comes out with mean square exactly 1 (a
    sum instead of a mean, a missing root or a missing square would all miss this)."""
    rng = np.random.default_rng(11)
    o = rng.standard_normal((7, 128)) * rng.uniform(0.01, 100.0, (7, 1))
    y = oracle.gated_rmsnorm(o, np.full(o.shape, 60.0), np.ones(128), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.sign(y) == np.sign(o))


def test_gated_rmsnorm_gate_values():
    """The gate is a logistic sigmoid of g itself: g = 0 halves the output exactly, a strongly negative
    g closes it, a strongly positive one leaves the normalised row (a sign slip swaps the last two)."""
    rng = np.random.default_rng(12)
    o, w = rng.standard_normal((5, 128)), rng.standard_normal(128)
    open_ = oracle.gated_rmsnorm(o, np.full(o.shape, 60.0), w, 1e-6)
    half = oracle.gated_rmsnorm(o, np.zeros(o.shape), w, 1e-6)
    shut = oracle.gated_rmsnorm(o, np.full(o.shape, -60.0), w, 1e-6)
    assert np.array_equal(half, 0.5 * open_)
    assert np.max(np.abs(shut)) < 1e-20 * np.max(np.abs(open_))
    g1 = np.log(3.0)  # sigmoid(ln 3) = 3/4
    q = oracle.gated_rmsnorm(o, np.full(o.shape, g1), w, 1e-6)
    assert np.allclose(q, 0.75 * open_, rtol=1e-15, atol=0)


def test_gated_rmsnorm_invariances():
    """Scale invariance at eps = 0 (RMSNorm ignores the row's magnitude), oddness in o, equivariance
    under a channel permutation of (o, g, w), and the weight acting per channel."""
    rng = np.random.default_rng(13)
    o, g, w = rng.standard_normal((6, 128)), rng.standard_normal((6, 128)), rng.standard_normal(128)
    y = oracle.gated_rmsnorm(o, g, w, 0.0)
    assert np.allclose(oracle.gated_rmsnorm(37.5 * o, g, w, 0.0), y, rtol=1e-13, atol=0)
    assert np.array_equal(oracle.gated_rmsnorm(-o, g, w, 0.0), -y)
    perm = rng.permutation(128)
    assert np.allclose(oracle.gated_rmsnorm(o[:, perm], g[:, perm], w[perm], 0.0), y[:, perm], rtol=1e-14, atol=0)
    w2 = w.copy()
    w2[5] *= 2.0
    y2 = oracle.gated_rmsnorm(o, g, w2, 0.0)
    assert np.array_equal(y2[:, 5], 2.0 * y[:, 5]) and np.array_equal(np.delete(y2, 5, 1), np.delete(y, 5, 1))


def test_gated_rmsnorm_eps():
    """eps sits inside the root and is added to the mean square: with eps = ms the row shrinks by
    exactly 1/sqrt(2); with eps far above ms the map becomes linear, o / sqrt(eps)."""
    rng = np.random.default_rng(14)
    o = rng.standard_normal((1, 128))
    ms = float(np.mean(o * o))
    g, w = np.full(o.shape, 60.0), np.ones(128)
    y0 = oracle.gated_rmsnorm(o, g, w, 0.0)
    assert np.allclose(oracle.gated_rmsnorm(o, g, w, ms), y0 / math.sqrt(2.0), rtol=1e-14, atol=0)
    big = 1e12
    assert np.allclose(oracle.gated_rmsnorm(o, g, w, big), o / math.sqrt(big), rtol=1e-9, atol=0)


# ---------------------------------------------------------------- the KDA prologue
# The pages name the fused operations (short conv on q/k/v with SiLU and the conv-state carry, beta's
# sigmoid) but give neither the conv width nor the decay-gate formula; these pin the oracle's reading:
# a causal depthwise conv whose tap j reads token t - W + 1 + j, SiLU, per-head L2 norm of q and k,
# beta = sigmoid, gk = -softplus, and a state that carries the last W - 1 raw rows.

def _prologue_case(rng, L, H, W, w=None):
    x = [rng.standard_normal((L, H, 128)) for _ in range(3)]
    cw = rng.standard_normal((3, H * 128, W)) if w is None else np.broadcast_to(w, (3, H * 128, W)).copy()
    st = rng.standard_normal((3, W - 1, H * 128))
    b, g = rng.standard_normal((L, H)), rng.standard_normal((L, H, 128))
    return x, cw, st, b, g


def test_prologue_taps_and_state():
    """Tap W-1 is the current token, tap 0 the token W-1 back (taken from the carried state for the
    first tokens); a reversed or shifted convolution fails one of the two."""
    rng = np.random.default_rng(31)
    L, H, W = 6, 1, 4
    silu = lambda c: c / (1.0 + np.exp(-c))
    x, _, st, b, g = _prologue_case(rng, L, H, W)
    now = np.zeros(W); now[W - 1] = 1.0
    _, _, v, _, _, _ = oracle.prologue(*x, np.broadcast_to(now, (3, 128, W)).copy(), st, b, g, 0.0)
    assert np.allclose(v, silu(x[2]), rtol=1e-14, atol=0)  # (numpy's exp and libm's may differ in the last bit)
    old = np.zeros(W); old[0] = 1.0
    _, _, v, _, _, _ = oracle.prologue(*x, np.broadcast_to(old, (3, 128, W)).copy(), st, b, g, 0.0)
    xv = x[2].reshape(L, 128)
    for t in range(L):
        src = xv[t - (W - 1)] if t >= W - 1 else st[2, t]  # state row t holds token t - (W - 1)
        assert np.allclose(v[t].reshape(128), silu(src), rtol=1e-14, atol=0)


def test_prologue_conv_sums_taps():
    """Weights (1, -1) on the two newest taps of a sequence that is constant in time (state included)
    give a zero pre-activation, so SiLU(0) = 0 exactly; changing one state row breaks it only where that
    row is read."""
    rng = np.random.default_rng(32)
    L, H, W = 5, 1, 3
    x, _, st, b, g = _prologue_case(rng, L, H, W)
    row = rng.standard_normal(128)
    xs = [np.broadcast_to(row, (L, 1, 128)).copy() for _ in range(3)]
    sts = np.broadcast_to(row, (3, W - 1, 128)).copy()
    w = np.array([0.0, -1.0, 1.0])
    _, _, v, _, _, _ = oracle.prologue(*xs, np.broadcast_to(w, (3, 128, W)).copy(), sts, b, g, 0.0)
    assert np.all(v == 0.0)
    sts[2, W - 2] += 1.0  # the newest carried row: read only by token 0's middle tap
    _, _, v, _, _, _ = oracle.prologue(*xs, np.broadcast_to(w, (3, 128, W)).copy(), sts, b, g, 0.0)
    assert np.all(v[0] != 0.0) and np.all(v[1:] == 0.0)


def test_prologue_norms_and_gates():
    """q and k come out with unit norm per (token, head) at eps = 0, v is not normalised; beta is the
    logistic sigmoid of its logit (1/2 at 0, 3/4 at ln 3) and exp(gk) = sigmoid(-g_raw), so gk <= 0."""
    rng = np.random.default_rng(33)
    L, H, W = 7, 3, 4
    x, cw, st, b, g = _prologue_case(rng, L, H, W)
    b[0, 0], b[0, 1] = 0.0, math.log(3.0)
    g[0, 0, :2] = (0.0, math.log(3.0))
    q, k, v, beta, gk, _ = oracle.prologue(*x, cw, st, b, g, 0.0)
    assert np.allclose(np.linalg.norm(q, axis=2), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(np.linalg.norm(k, axis=2), 1.0, rtol=0, atol=1e-14)
    assert not np.allclose(np.linalg.norm(v, axis=2), 1.0)
    assert beta[0, 0] == 0.5 and abs(beta[0, 1] - 0.75) < 1e-15
    assert abs(gk[0, 0, 0] + math.log(2.0)) < 1e-15 and abs(gk[0, 0, 1] + math.log(4.0)) < 1e-15
    assert np.all(gk <= 0) and np.allclose(np.exp(gk), 1.0 / (1.0 + np.exp(g)), rtol=1e-14, atol=0)
    # eps sits inside the root, added to the sum of squares: eps = |u|^2 of a row shrinks it by 1/sqrt(2)
    uk = k[2, 1]  # the unit row at eps = 0
    _, _, vk, _, _, _ = oracle.prologue(x[1], x[1], x[1], cw[[1, 1, 1]], st[[1, 1, 1]], b, g, 0.0)
    ek = float(np.sum(vk[2, 1] ** 2))  # |u|^2 of k's row
    _, k3, _, _, _, _ = oracle.prologue(*x, cw, st, b, g, ek)
    assert np.allclose(k3[2, 1], uk / math.sqrt(2.0), rtol=1e-13, atol=0)


def test_prologue_state_carry():
    """Running a sequence in two calls, the first call's state_out feeding the second, gives the same
    outputs and final state as one call (all W in 1..5, split points inside the first W - 1 tokens)."""
    rng = np.random.default_rng(34)
    for W in (1, 2, 3, 4, 5):
        L, H = 9, 2
        x, cw, st, b, g = _prologue_case(rng, L, H, W)
        full = oracle.prologue(*x, cw, st, b, g, 1e-6)
        for m in (0, 1, W - 1, 5, L):
            m = max(0, min(L, m))
            a = oracle.prologue(*(t[:m] for t in x), cw, st, b[:m], g[:m], 1e-6)
            c = oracle.prologue(*(t[m:] for t in x), cw, a[5], b[m:], g[m:], 1e-6)
            for i in range(5):
                assert np.array_equal(np.concatenate([a[i], c[i]]), full[i])
            assert np.array_equal(c[5], full[5])
