"""Pins of the fp64 oracle against what the pages and the mathematics fix.

CPU only. Each test ties the oracle to something other than itself: a hand
case, a closed form, the pages' hidden-attention form, a library routine, or
an invariant the definition implies. A plausible mistake (dropped D term,
wrong sign of A, off-by-one in the decay, transposed state, wrong norm
placement, missing gate) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from state_space_model_sscan_amd import inputs as gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def softplus_np(v):
    # independent of the oracle's form: log(1 + e^v) via logaddexp
    return np.logaddexp(0.0, v)


def sigmoid_np(z):
    return 0.5 * (1.0 + np.tanh(0.5 * z))


# --------------------------------------------------------------- hand cases
def _hand_inputs(case):
    L = case["seq"]
    v = case["dt_raw"]
    dt_raw = math.log(math.e - 1.0) if v == "ln(e-1)" else float(v)
    x = np.array(case["x"], float).reshape(1, L, 1)
    return dict(
        x=x,
        dt_raw=np.full((1, L, 1), dt_raw),
        dt_bias=np.array([case["dt_bias"]]),
        A_log=np.array([[case["A_log"]]]),
        B=np.full((1, L, 1, 1), case["B"]),
        C=np.full((1, L, 1, 1), case["C"]),
        D=np.array([case["D"]]),
    )


def test_hand_case_halving():
    case = json.load(open(os.path.join(GOLD, "mamba1_hand_cases.json")))["cases"][0]
    a = _hand_inputs(case)
    y, h, _ = oracle.mamba1(**a)
    want = math.log(2.0) * np.array(case["y_over_ln2"])
    np.testing.assert_allclose(y[0, :, 0], want, rtol=1e-15, atol=0)
    assert abs(h[0, 0, 0] - want[-1]) < 1e-15  # y = C.h with C = 1, D = 0


def test_hand_case_impulse_decay_and_D():
    case = json.load(open(os.path.join(GOLD, "mamba1_hand_cases.json")))["cases"][1]
    a = _hand_inputs(case)
    y, h, _ = oracle.mamba1(**a)
    t = np.arange(4)
    want = 6.0 * np.exp(-t) + 0.5 * np.array(case["x"], float)
    np.testing.assert_allclose(y[0, :, 0], want, rtol=1e-14)
    np.testing.assert_allclose(h[0, 0, 0], 2.0 * math.exp(-3), rtol=1e-14)


def test_gate_closed_forms():
    case = json.load(open(os.path.join(GOLD, "mamba1_hand_cases.json")))["cases"][0]
    a = _hand_inputs(case)
    y, _, _ = oracle.mamba1(**a)
    # z = 0: silu(0) = 0 silences the token
    y0, _, _ = oracle.mamba1(**a, z=np.zeros((1, 4, 1)))
    assert np.all(y0 == 0.0)
    # z = 1: y * sigmoid(1) = y * e / (1 + e)
    y1, _, _ = oracle.mamba1(**a, z=np.ones((1, 4, 1)))
    np.testing.assert_allclose(y1, y * (math.e / (1 + math.e)), rtol=1e-15)
    # z = 40: silu(40) = 40 to double precision
    y40, _, _ = oracle.mamba1(**a, z=np.full((1, 4, 1), 40.0))
    np.testing.assert_allclose(y40, 40.0 * y, rtol=1e-15)


def test_softplus_special_values():
    # dt_raw = -inf is a zero step (softplus(-inf) = 0): the state passes unchanged
    a = dict(x=np.ones((1, 2, 1)), dt_raw=np.array([[[0.0]], [[-np.inf]]]).reshape(1, 2, 1),
             dt_bias=np.zeros(1), A_log=np.zeros((1, 1)), B=np.ones((1, 2, 1, 1)),
             C=np.ones((1, 2, 1, 1)), D=np.zeros(1))
    y, h, st = oracle.mamba1(**a, want_states=True)
    assert st[0, 1, 0, 0] == st[0, 0, 0, 0] == math.log(2.0)
    assert y[0, 1, 0] == y[0, 0, 0]


# --------------------------------------------------------- closed forms
def _rand_m1(rng, b, L, Dc, N, G=1, h0=True):
    return dict(
        x=rng.standard_normal((b, L, Dc)),
        dt_raw=0.5 * rng.standard_normal((b, L, Dc)),
        dt_bias=rng.uniform(-4, -1, Dc),
        A_log=np.log(rng.uniform(1, 16, (Dc, N))),
        B=rng.standard_normal((b, L, G, N)),
        C=rng.standard_normal((b, L, G, N)),
        D=rng.uniform(0.5, 1.5, Dc),
        h0=0.1 * rng.standard_normal((b, Dc, N)) if h0 else None,
    )


def test_s4_time_invariant_closed_form():
    """Constant dt, B, C: y_t = sum_n C_n (Abar_n^(t+1) h0_n + sum_k Abar_n^k dt B_n x_(t-k)) + D x_t
    ('Mamba' tokentrails, step 'The scan': h_t = Abar h_(t-1) + Bbar x_t, y_t = C h_t)."""
    rng = np.random.default_rng(1)
    b, L, Dc, N = 2, 40, 3, 5
    a = _rand_m1(rng, b, L, Dc, N)
    # constant over tokens
    a["dt_raw"] = np.broadcast_to(a["dt_raw"][:, :1, :], (b, L, Dc)).copy()
    a["B"] = np.broadcast_to(a["B"][:, :1], (b, L, 1, N)).copy()
    a["C"] = np.broadcast_to(a["C"][:, :1], (b, L, 1, N)).copy()
    y, h, _ = oracle.mamba1(**a)
    dt = softplus_np(a["dt_raw"][:, 0, :] + a["dt_bias"])        # [b, Dc]
    A = -np.exp(a["A_log"])                                      # [Dc, N]
    Abar = np.exp(dt[:, :, None] * A[None])                      # [b, Dc, N]
    Bn, Cn = a["B"][:, 0, 0], a["C"][:, 0, 0]                    # [b, N]
    want = np.zeros((b, L, Dc))
    for t in range(L):
        k = np.arange(t + 1)
        powk = Abar[:, :, :, None] ** k                          # [b, Dc, N, t+1]
        xs = a["x"][:, t - k, :]                                 # [b, t+1, Dc]
        conv = np.einsum("bn,bcnk,bkc->bc", Cn * 1.0, powk * (dt[:, :, None, None] * Bn[:, None, :, None]), xs)
        init = np.einsum("bn,bcn,bcn->bc", Cn, Abar ** (t + 1), a["h0"])
        want[:, t] = conv + init + a["D"] * a["x"][:, t]
    np.testing.assert_allclose(y, want, rtol=1e-10, atol=1e-12)


def _mamba1_hidden_attention(a, bc_eps=0.0, z=None):
    """y_t = sum_{s<=t} sum_n C_t[n] B_s[n] exp(A_n * sum_{k=s+1..t} dt_k) dt_s x_s
             + sum_n C_t[n] exp(A_n * sum_{k<=t} dt_k) h0[n] + D x_t
    ('Falcon-Mamba', section 'The mixer's values': the hidden attention of the Mamba page
    rebuilds the scan's output)."""
    x, B, C = a["x"], a["B"][:, :, 0], a["C"][:, :, 0]
    if bc_eps > 0:
        B = B / np.sqrt(np.mean(B * B, -1, keepdims=True) + bc_eps)
        C = C / np.sqrt(np.mean(C * C, -1, keepdims=True) + bc_eps)
    b, L, Dc = x.shape
    dt = softplus_np(a["dt_raw"] + a["dt_bias"])                 # [b, L, Dc]
    A = -np.exp(a["A_log"])                                      # [Dc, N]
    S = np.cumsum(dt, axis=1)                                    # inclusive
    y = np.zeros((b, L, Dc))
    for t in range(L):
        diff = S[:, t:t + 1, :] - S[:, : t + 1, :]               # [b, s, Dc]  sum_{k=s+1..t} dt_k
        dec = np.exp(diff[..., None] * A[None, None])            # [b, s, Dc, N]
        w = np.einsum("bn,bsn,bscn->bsc", C[:, t], B[:, : t + 1], dec)
        y[:, t] = np.einsum("bsc,bsc,bsc->bc", w, dt[:, : t + 1], x[:, : t + 1])
        if a.get("h0") is not None:
            y[:, t] += np.einsum("bn,bcn,bcn->bc", C[:, t], np.exp(S[:, t, :, None] * A[None]), a["h0"])
        y[:, t] += a["D"] * x[:, t]
    if z is not None:
        y = y * z * sigmoid_np(z)
    return y


def test_mamba1_hidden_attention_form():
    rng = np.random.default_rng(2)
    a = _rand_m1(rng, 2, 33, 4, 6)
    y, _, _ = oracle.mamba1(**a)
    np.testing.assert_allclose(y, _mamba1_hidden_attention(a), rtol=1e-10, atol=1e-12)


def test_mamba1_hidden_attention_with_gate_and_bcnorm():
    rng = np.random.default_rng(3)
    a = _rand_m1(rng, 1, 21, 3, 16)
    z = rng.standard_normal((1, 21, 3))
    y, _, _ = oracle.mamba1(**a, z=z, bc_eps=1e-6)
    np.testing.assert_allclose(y, _mamba1_hidden_attention(a, 1e-6, z), rtol=1e-10, atol=1e-12)


def _ssd_hidden_attention(s):
    """y_t for every head from the pages' statement of the Mamba-2 hidden attention
    ('Mamba-2', section 'The hidden attention'): token t reads token s <= t through the
    weight (C_t . B_s) * exp(decays_{s+1} + ... + decays_t) * betas_s, with
    betas = softplus(dt_raw + dt_bias), decays = betas * A and head h reading group
    h // (H / G) ('The mixer's values'); y_t = sum of the weighted x_s + D x_t, the entering
    state reaches token t decayed by every decay up to t and read through C_t, then the gate.
    Written as plain loops over (t, s), the decay sum formed for each pair."""
    x, B, C = s["x"], s["B"], s["C"]
    b, L, H, P = x.shape
    G = B.shape[2]
    per_group = H // G
    betas = softplus_np(s["dt_raw"] + s["dt_bias"])
    A = -np.exp(s["A_log"])
    y = np.zeros((b, L, H, P))
    for bi in range(b):
        for h in range(H):
            g = h // per_group
            for t in range(L):
                acc = s["D"][h] * x[bi, t, h]
                for src in range(t + 1):
                    decay_sum = sum(betas[bi, k, h] * A[h] for k in range(src + 1, t + 1))
                    weight = np.dot(C[bi, t, g], B[bi, src, g]) * np.exp(decay_sum) * betas[bi, src, h]
                    acc = acc + weight * x[bi, src, h]
                if s.get("h0") is not None:
                    carried = np.exp(sum(betas[bi, k, h] * A[h] for k in range(t + 1)))
                    acc = acc + carried * (s["h0"][bi, h] @ C[bi, t, g])
                y[bi, t, h] = acc
    if s.get("z") is not None:
        y = y * s["z"] * sigmoid_np(s["z"])
    return y


def _rand_ssd(rng, b, L, H, P, N, G=1, h0=True, z=False):
    return dict(
        x=rng.standard_normal((b, L, H, P)),
        dt_raw=0.5 * rng.standard_normal((b, L, H)),
        dt_bias=rng.uniform(-4, -1, H),
        A_log=np.log(rng.uniform(1, 16, H)),
        B=rng.standard_normal((b, L, G, N)),
        C=rng.standard_normal((b, L, G, N)),
        D=rng.uniform(0.5, 1.5, H),
        z=rng.standard_normal((b, L, H, P)) if z else None,
        h0=0.1 * rng.standard_normal((b, H, P, N)) if h0 else None,
    )


@pytest.mark.parametrize("G", [1, 2])
def test_ssd_hidden_attention_form(G):
    rng = np.random.default_rng(4)
    s = _rand_ssd(rng, 2, 29, 4, 3, 8, G=G, z=True)
    y, _, _ = oracle.ssd(**s)
    np.testing.assert_allclose(y, _ssd_hidden_attention(s), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("G", [1, 2])
def test_ssd_attention_rebuilds_the_scan(G):
    """The oracle's hidden attention map, applied to x, gives the token loop's y
    before the gate ('Mamba-2', section 'The hidden attention'): two code paths."""
    rng = np.random.default_rng(7 + G)
    s = _rand_ssd(rng, 2, 23, 4, 3, 8, G=G, h0=False)
    s["dt_raw"][0, 5, :] = -np.inf  # a zero step: its column of the map is zero
    alpha = oracle.ssd_attention(s["dt_raw"], s["dt_bias"], s["A_log"], s["B"], s["C"])
    y, _, _ = oracle.ssd(**s)
    y2 = np.einsum("btsh,bshp->bthp", alpha, s["x"]) + s["D"][None, None, :, None] * s["x"]
    np.testing.assert_allclose(y2, y, rtol=1e-10, atol=1e-12)
    assert np.all(alpha[0, :, 5, :] == 0.0)
    # causal: nothing above the diagonal
    L = alpha.shape[1]
    assert np.all(alpha[:, np.triu_indices(L, 1)[0], np.triu_indices(L, 1)[1], :] == 0.0)


def test_ssd_attention_hand_case():
    """One head, state_dim 1, three tokens, written out: alpha[t, s] = C_t B_s exp(sum of the
    decays after s up to t) beta_s, with beta = softplus(dt), decay = beta * A."""
    sp = lambda v: math.log1p(math.exp(v))
    dt_raw = np.array([[[0.0], [0.5], [-1.0]]])
    dt_bias = np.array([0.25])
    A_log = np.array([math.log(2.0)])  # A = -2
    B = np.array([[[[1.5]], [[-2.0]], [[0.5]]]])
    C = np.array([[[[0.5]], [[3.0]], [[-1.0]]]])
    beta = [sp(0.25), sp(0.75), sp(-0.75)]
    alpha = oracle.ssd_attention(dt_raw, dt_bias, A_log, B, C)[0, :, :, 0]
    want = np.zeros((3, 3))
    Bv, Cv = [1.5, -2.0, 0.5], [0.5, 3.0, -1.0]
    for t in range(3):
        for s_ in range(t + 1):
            dec = sum(-2.0 * beta[k] for k in range(s_ + 1, t + 1))
            want[t, s_] = Cv[t] * Bv[s_] * math.exp(dec) * beta[s_]
    np.testing.assert_allclose(alpha, want, rtol=1e-14, atol=0)
    assert alpha[2, 0] == pytest.approx(-1.0 * 1.5 * math.exp(-2.0 * (beta[1] + beta[2])) * beta[0], rel=1e-14)


def test_ssd_equals_mamba1_with_tied_A():
    """Mamba-2 is Mamba-1 with one decay per head: channel (h, p), dt broadcast over p,
    A[c, n] = A_h, D[c] = D_h ('Mamba-2', section 'The mixer's values')."""
    rng = np.random.default_rng(5)
    b, L, H, P, N = 2, 25, 3, 4, 6
    s = _rand_ssd(rng, b, L, H, P, N, z=True)
    y2, h2, st2 = oracle.ssd(**s, want_states=True)
    Dc = H * P
    m = dict(
        x=s["x"].reshape(b, L, Dc),
        dt_raw=np.repeat(s["dt_raw"], P, axis=2),
        dt_bias=np.repeat(s["dt_bias"], P),
        A_log=np.repeat(np.repeat(s["A_log"], P)[:, None], N, axis=1),
        B=s["B"], C=s["C"], D=np.repeat(s["D"], P),
        z=s["z"].reshape(b, L, Dc),
        h0=s["h0"].reshape(b, Dc, N),
    )
    y1, h1, st1 = oracle.mamba1(**m, want_states=True)
    np.testing.assert_allclose(y1.reshape(y2.shape), y2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(h1.reshape(h2.shape), h2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st1.reshape(st2.shape), st2, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------- state invariants
def test_states_last_equals_state_output_bitwise():
    rng = np.random.default_rng(6)
    a = _rand_m1(rng, 2, 17, 5, 4)
    _, h, st = oracle.mamba1(**a, want_states=True)
    assert np.array_equal(st[:, -1], h)
    s = _rand_ssd(rng, 2, 17, 3, 4, 5)
    _, h, st = oracle.ssd(**s, want_states=True)
    assert np.array_equal(st[:, -1], h)


@pytest.mark.parametrize("cut", [1, 8, 19])
def test_split_sequence_equals_whole(cut):
    """Scanning [0, cut) and then [cut, L) from the first part's state equals the whole scan
    ('Mamba', section 'The state': the state is handed from state_output to state_input)."""
    rng = np.random.default_rng(7)
    L = 20
    a = _rand_m1(rng, 2, L, 4, 3)
    z = rng.standard_normal((2, L, 4))
    y, h, _ = oracle.mamba1(**a, z=z)

    def part(lo, hi, h0):
        p = dict(a)
        for k in ("x", "dt_raw", "B", "C"):
            p[k] = a[k][:, lo:hi]
        p["h0"] = h0
        return oracle.mamba1(**p, z=z[:, lo:hi])

    ya, ha, _ = part(0, cut, a["h0"])
    yb, hb, _ = part(cut, L, ha)
    assert np.array_equal(np.concatenate([ya, yb], 1), y)
    assert np.array_equal(hb, h)
    # SSD, same property
    s = _rand_ssd(rng, 2, L, 3, 2, 4, z=True)
    y, h, _ = oracle.ssd(**s)

    def spart(lo, hi, h0):
        p = dict(s)
        for k in ("x", "dt_raw", "B", "C", "z"):
            p[k] = s[k][:, lo:hi]
        p["h0"] = h0
        return oracle.ssd(**p)

    ya, ha, _ = spart(0, cut, s["h0"])
    yb, hb, _ = spart(cut, L, ha)
    assert np.array_equal(np.concatenate([ya, yb], 1), y)
    assert np.array_equal(hb, h)


def test_one_token_steps_equal_prompt():
    """A prompt of L tokens equals L one-token calls chained through the state (the decode
    step: update first, then read; 'Mamba', section 'The state')."""
    rng = np.random.default_rng(8)
    L = 9
    a = _rand_m1(rng, 3, L, 4, 5)
    y, h, _ = oracle.mamba1(**a)
    state = a["h0"]
    for t in range(L):
        p = dict(a)
        for k in ("x", "dt_raw", "B", "C"):
            p[k] = a[k][:, t:t + 1]
        p["h0"] = state
        yt, state, _ = oracle.mamba1(**p)
        assert np.array_equal(yt[:, 0], y[:, t])
    assert np.array_equal(state, h)


def test_state_layout_is_read_through_C():
    """With C = e_m at the last token, D = 0 and no gate, y_last reads state entry m: this ties
    the stored layout ([b, channels, N] and [b, H, P, N]) to the readout y = C . h."""
    rng = np.random.default_rng(9)
    a = _rand_m1(rng, 2, 6, 5, 7)
    a["D"] = np.zeros(5)
    m = 3
    a["C"][:, -1] = 0.0
    a["C"][:, -1, 0, m] = 1.0
    y, h, _ = oracle.mamba1(**a)
    np.testing.assert_allclose(y[:, -1, :], h[:, :, m], rtol=1e-15)
    s = _rand_ssd(rng, 2, 6, 3, 4, 7)
    s["D"] = np.zeros(3)
    s["C"][:, -1] = 0.0
    s["C"][:, -1, 0, m] = 1.0
    y, h, _ = oracle.ssd(**s)
    np.testing.assert_allclose(y[:, -1], h[:, :, :, m], rtol=1e-15)


def test_zero_step_is_exact():
    """A zero step writes nothing and does not decay the state, bit for bit
    ('Mamba-2', section 'A zero step skips a token exactly')."""
    rng = np.random.default_rng(10)
    a = _rand_m1(rng, 2, 8, 4, 5)
    a["dt_raw"][:, 3] = -np.inf
    _, _, st = oracle.mamba1(**a, want_states=True)
    assert np.array_equal(st[:, 3], st[:, 2])
    s = _rand_ssd(rng, 2, 8, 3, 4, 5)
    s["dt_raw"][:, 3] = -np.inf
    _, _, st = oracle.ssd(**s, want_states=True)
    assert np.array_equal(st[:, 3], st[:, 2])


# --------------------------------------------------------- B/C norm
def test_bc_norm_rms_of_one_and_direction():
    """The scan reads B / rms(B): one token from a zero state gives h = dt * x * B_normed,
    whose RMS is one and whose direction is B's ('Falcon-Mamba', section 'Where the norms sit')."""
    rng = np.random.default_rng(11)
    N = 16
    a = dict(x=np.full((1, 1, 1), 1.7), dt_raw=np.zeros((1, 1, 1)), dt_bias=np.zeros(1),
             A_log=np.zeros((1, N)), B=3.0 * rng.standard_normal((1, 1, 1, N)),
             C=rng.standard_normal((1, 1, 1, N)), D=np.zeros(1))
    eps = 1e-6
    _, h, _ = oracle.mamba1(**a, bc_eps=eps)
    bn = h[0, 0] / (math.log(2.0) * 1.7)
    rms = math.sqrt(np.mean(bn * bn))
    ms = np.mean(a["B"][0, 0, 0] ** 2)
    assert abs(rms - 1.0) <= eps / (2 * ms) + 1e-13
    cos = bn @ a["B"][0, 0, 0] / (np.linalg.norm(bn) * np.linalg.norm(a["B"][0, 0, 0]))
    assert abs(cos - 1.0) < 1e-14


def test_bc_norm_scale_invariance():
    rng = np.random.default_rng(12)
    a = _rand_m1(rng, 1, 12, 3, 16)
    y1, h1, _ = oracle.mamba1(**a, bc_eps=1e-30)
    b = dict(a)
    b["B"] = 5.0 * a["B"]
    b["C"] = 0.25 * a["C"]
    y2, h2, _ = oracle.mamba1(**b, bc_eps=1e-30)
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(h2, h1, rtol=1e-12, atol=1e-14)
    # and without the norm the scaling shows
    y3, _, _ = oracle.mamba1(**b)
    y4, _, _ = oracle.mamba1(**a)
    assert not np.allclose(y3, y4)


# --------------------------------------------------------- derived invariants
def test_linearity_in_x_and_h0():
    rng = np.random.default_rng(13)
    a1 = _rand_m1(rng, 2, 15, 4, 5)
    a2 = dict(a1)
    a2["x"] = rng.standard_normal(a1["x"].shape)
    a2["h0"] = rng.standard_normal(a1["h0"].shape)
    al, be = 0.7, -1.3
    a3 = dict(a1)
    a3["x"] = al * a1["x"] + be * a2["x"]
    a3["h0"] = al * a1["h0"] + be * a2["h0"]
    y1, h1, _ = oracle.mamba1(**a1)
    y2, h2, _ = oracle.mamba1(**a2)
    y3, h3, _ = oracle.mamba1(**a3)
    np.testing.assert_allclose(y3, al * y1 + be * y2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(h3, al * h1 + be * h2, rtol=1e-11, atol=1e-12)
    # zero input and zero state stay zero
    a0 = dict(a1)
    a0["x"] = np.zeros_like(a1["x"])
    a0["h0"] = None
    y0, h0, _ = oracle.mamba1(**a0)
    assert not y0.any() and not h0.any()


def test_batch_independence_and_channel_permutation():
    rng = np.random.default_rng(14)
    a = _rand_m1(rng, 3, 10, 6, 4)
    y, h, _ = oracle.mamba1(**a)
    one = {k: (v[1:2] if k in ("x", "dt_raw", "B", "C", "h0") else v) for k, v in a.items()}
    y1, h1, _ = oracle.mamba1(**one)
    assert np.array_equal(y1[0], y[1]) and np.array_equal(h1[0], h[1])
    perm = rng.permutation(6)
    ap = dict(a)
    for k in ("x", "dt_raw"):
        ap[k] = a[k][:, :, perm]
    ap["dt_bias"], ap["A_log"], ap["D"] = a["dt_bias"][perm], a["A_log"][perm], a["D"][perm]
    ap["h0"] = a["h0"][:, perm]
    yp, hp, _ = oracle.mamba1(**ap)
    assert np.array_equal(yp, y[:, :, perm]) and np.array_equal(hp, h[:, perm])


def test_printed_shapes_of_a_ten_token_prompt():
    """'Mamba' (nnterp guide): a 10-token prompt on mamba-130m has x [1,10,1536], B and C
    [1,10,1,16], state [1,1536,16], states [1,10,1536,16]; a decode step's y is [1,1,1536]."""
    inp = gen.make_mamba1(1, 10, 1536, 16, act="f32", seed=3, gate=True, want_states=True)
    y, h, st = oracle.run_inputs(inp)
    assert inp.B.shape == (1, 10, 1, 16) and inp.x.shape == (1, 10, 1536)
    assert y.shape == (1, 10, 1536) and h.shape == (1, 1536, 16) and st.shape == (1, 10, 1536, 16)
    step = gen.make_mamba1(1, 1, 1536, 16, act="f32", seed=4, h0=True)
    y1, h1, _ = oracle.run_inputs(step)
    assert y1.shape == (1, 1, 1536) and h1.shape == (1, 1536, 16)


# --------------------------------------------------------- the steps around the scan
def test_conv1d_silu_against_torch_conv1d():
    """Causal depthwise conv (width 4, padding 3, first L outputs) then silu, as torch's Conv1d."""
    rng = np.random.default_rng(15)
    b, L, Dc, W = 2, 13, 5, 4
    x = rng.standard_normal((b, L, Dc))
    w = rng.standard_normal((Dc, W))
    bias = rng.standard_normal(Dc)
    out, st = oracle.conv1d_silu(x, w, bias)
    xt = torch.from_numpy(x).permute(0, 2, 1)
    ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :], torch.from_numpy(bias),
                                     padding=W - 1, groups=Dc)[..., :L]
    ref = torch.nn.functional.silu(ref).permute(0, 2, 1).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(st, x[:, -(W - 1):, :].transpose(0, 2, 1))
    # continuation from the conv state equals the whole
    oa, sa = oracle.conv1d_silu(x[:, :6], w, bias)
    ob, sb = oracle.conv1d_silu(x[:, 6:], w, bias, sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob], 1), out)
    np.testing.assert_array_equal(sb, st)


def test_gated_rmsnorm_against_torch():
    rng = np.random.default_rng(16)
    y = rng.standard_normal((7, 24))
    z = rng.standard_normal((7, 24))
    w = rng.uniform(0.5, 2, 24)
    out = oracle.gated_rmsnorm(y, z, w, 1e-5)
    g = torch.from_numpy(y) * torch.nn.functional.silu(torch.from_numpy(z))
    ref = torch.nn.functional.rms_norm(g, (24,), torch.from_numpy(w), 1e-5).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------- generator
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(17)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    v[:4] = [np.inf, -np.inf, 0.0, -0.0]
    ours = gen.bf16_round(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    bits = gen.bf16_bits(ours)
    assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy(), ours)


def test_generator_is_deterministic_and_in_regime():
    a = gen.make_mamba1(2, 64, 256, 16, act="bf16", seed=5, gate=True)
    b = gen.make_mamba1(2, 64, 256, 16, act="bf16", seed=5, gate=True)
    for k in ("x", "dt_raw", "B", "C", "z", "dt_bias", "D"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert np.array_equal(gen.bf16_round(a.x), a.x)
    # dt_bias is an inverse softplus of values in [1e-3, 1e-1]
    sp = softplus_np(a.dt_bias.astype(np.float64))
    assert sp.min() >= 1e-3 * 0.999 and sp.max() <= 1e-1 * 1.001
    # median retained fraction exp(dt*A) near the pages' 0.89 on real weights (a sanity check)
    dt = softplus_np(a.dt_raw.astype(np.float64) + a.dt_bias)
    keep = np.exp(dt[..., None] * -np.exp(a.A_log.astype(np.float64)))
    assert 0.8 < np.median(keep) < 0.98
