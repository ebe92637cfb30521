"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle on
the same seeded inputs. Small cases compare every element; the full-size
workloads compare a spread of sampled channels/heads over the whole sequence."""
import numpy as np
import pytest
import torch

import oracle
from state_space_model_sscan_amd import binding as bd
from state_space_model_sscan_amd import inputs as gen

from _gpu import (check, dev, host, mamba1_subset, par, run_mamba1, run_ssd, sample_channels, say,
                  ssd_subset)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


# ------------------------------------------------------------ Mamba-1, small
M1_CASES = [
    # batch, seqlen, channels, N, act, gate, h0, states, bc_eps
    (1, 1, 64, 16, "f32", False, False, True, 0.0),
    (1, 2, 100, 16, "f32", True, True, True, 0.0),
    (3, 3, 64, 16, "bf16", True, False, False, 0.0),
    (2, 63, 200, 16, "f32", True, True, False, 1e-6),
    (2, 64, 128, 16, "bf16", False, True, True, 0.0),
    (1, 65, 64, 5, "f32", True, False, True, 0.0),
    (3, 255, 96, 16, "bf16", True, True, False, 1e-6),
    (1, 256, 64, 8, "f32", False, False, False, 0.0),
    (2, 257, 130, 32, "f32", True, True, True, 0.0),
    (1, 1000, 64, 16, "f32", True, True, False, 1e-5),
    (2, 1000, 192, 16, "bf16", True, False, False, 0.0),
    (1, 777, 64, 64, "f32", True, True, False, 0.0),
    (2, 3000, 64, 16, "f32", True, True, True, 0.0),     # several slices
    (16, 100, 4096, 16, "bf16", True, False, False, 0.0),  # one lane per channel
    (8, 77, 4096, 16, "f32", False, True, True, 1e-6),     # two lanes per channel
    (8, 45, 4096, 32, "f32", True, True, False, 0.0),      # 32 states, two lanes per channel
    (3, 333, 256, 64, "bf16", True, True, True, 0.0),      # 64 states, four lanes per channel
    (2, 300, 64, 128, "bf16", True, True, True, 1e-6),     # 128 states: the token loop
    (1, 129, 96, 100, "f32", True, False, False, 0.0),     # 100 of a padded 128
    (1, 3000, 64, 128, "f32", True, True, False, 0.0),     # 128 states, several slices
]


@pytest.mark.parametrize("case", M1_CASES, ids=lambda c: "b%d_L%d_D%d_N%d_%s_g%d_h%d_s%d_e%g" % c)
def test_mamba1_small(case):
    b, L, Dc, N, act, gate, h0, states, eps = case
    say("mamba1 case", case)
    inp = gen.make_mamba1(b, L, Dc, N, act=act, seed=L * 7 + Dc, gate=gate, h0=h0, bc_eps=eps,
                          want_states=states)
    yr, hr, sr = oracle.run_inputs(inp)
    yg, hg, sg = run_mamba1(inp)
    check(yg, yr, act, "y")
    check(hg, hr, act, "state_output")
    if states:
        check(sg, sr, act, "states")
        assert np.array_equal(sg[:, -1], hg), "states[:, -1] must equal state_output bit for bit"


# The plan gives state_dim 16/32/64 (with channels in groups of 4) to the
# row-per-channel kernel; these cases force the 1/2/4-lanes-per-channel kernel,
# which the other shapes take, through its tuning override.
LANE_CASES = [
    # lanes, batch, seqlen, channels, N, act, gate, h0, states, bc_eps
    (1, 2, 300, 256, 16, "bf16", True, True, False, 1e-6),
    (2, 3, 129, 192, 32, "f32", True, False, True, 0.0),
    (4, 2, 1000, 128, 16, "f32", False, True, False, 0.0),
    (4, 1, 77, 64, 64, "bf16", True, True, True, 1e-5),
]


@pytest.mark.parametrize("case", LANE_CASES, ids=lambda c: "K%d_b%d_L%d_D%d_N%d_%s_g%d_h%d_s%d_e%g" % c)
def test_mamba1_forced_lanes(case, monkeypatch):
    K, b, L, Dc, N, act, gate, h0, states, eps = case
    say("mamba1 forced lanes", case)
    monkeypatch.setenv("SSCAN_M1_LANES", str(K))
    inp = gen.make_mamba1(b, L, Dc, N, act=act, seed=L * 5 + Dc + K, gate=gate, h0=h0, bc_eps=eps,
                          want_states=states)
    yr, hr, sr = oracle.run_inputs(inp)
    yg, hg, sg = run_mamba1(inp)
    check(yg, yr, act, "y")
    check(hg, hr, act, "state_output")
    if states:
        check(sg, sr, act, "states")
        assert np.array_equal(sg[:, -1], hg)


def test_mamba1_grouped_B_C():
    inp = gen.make_mamba1(2, 300, 256, 16, ngroups=2, act="f32", seed=11, gate=True, h0=True)
    yr, hr, _ = oracle.run_inputs(inp)
    yg, hg, _ = run_mamba1(inp)
    check(yg, yr, "f32", "y")
    check(hg, hr, "f32", "state_output")


# ------------------------------------------------------------ the five workloads
def test_workload0_full():
    inp = gen.make_workload(0)
    say("workload 0", gen.WORKLOADS[0]["name"])
    yr, hr, sr = oracle.run_inputs(inp)
    yg, hg, sg = run_mamba1(inp)
    check(yg, yr, "f32", "y")
    check(hg, hr, "f32", "state_output")
    check(sg, sr, "f32", "states")
    assert np.array_equal(sg[:, -1], hg)


@pytest.mark.parametrize("wid", [1, 3])
def test_mamba1_workload_full_size_sampled(wid):
    inp = gen.make_workload(wid)
    say("workload", wid, gen.WORKLOADS[wid]["name"])
    yg, hg, _ = run_mamba1(inp)
    sel = sample_channels(inp.channels, 96, seed=wid)
    sub = mamba1_subset(inp, sel)
    yr, hr, _ = oracle.run_inputs(sub)
    check(yg[:, :, sel], yr, inp.act, "y")
    check(hg[:, sel], hr, inp.act, "state_output")


def test_workload2_fwd_and_512_steps():
    inp = gen.make_workload(2)
    say("workload 2", gen.WORKLOADS[2]["name"])
    yr, hr, _ = oracle.run_inputs(inp)
    yf, hf, _ = run_mamba1(inp)
    check(yf, yr, "f32", "y (fwd)")
    check(hf, hr, "f32", "state (fwd)")
    # the same sequence as 512 one-token calls, the state updated in place
    x, dt, z = dev(inp.x, "f32"), dev(inp.dt_raw, "f32"), dev(inp.z, "f32")
    B, C = dev(inp.B, "f32"), dev(inp.C, "f32")
    bias, alog, D = par(inp.dt_bias), par(inp.A_log), par(inp.D)
    state = par(inp.h0).clone()
    ys = torch.empty_like(x)
    for t in range(inp.seqlen):
        y1, _ = bd.sscan_step(state, x[:, t:t + 1].contiguous(), dt[:, t:t + 1].contiguous(), bias, alog,
                              B[:, t:t + 1].contiguous(), C[:, t:t + 1].contiguous(), D,
                              z[:, t:t + 1].contiguous(), state_output=state)
        ys[:, t] = y1[:, 0]
    torch.cuda.synchronize()
    ysh, hsh = host(ys), host(state)
    check(ysh, yr, "f32", "y (steps)")
    check(hsh, hr, "f32", "state (steps)")
    # fwd and steps against each other, scaled by the oracle's max
    assert np.max(np.abs(ysh - yf)) <= 1e-4 * np.max(np.abs(yr))
    assert np.max(np.abs(hsh - hf)) <= 1e-4 * np.max(np.abs(hr))


def test_workload4_ssd_full_size_sampled():
    inp = gen.make_workload(4)
    say("workload 4", gen.WORKLOADS[4]["name"])
    yg, hg, _ = run_ssd(inp)
    heads = np.array([0, 1, 37, 78, 79])
    sub = ssd_subset(inp, heads)
    yr, hr, _ = oracle.run_inputs(sub)
    check(yg[:, :, heads], yr, "bf16", "y")
    check(hg[:, heads], hr, "bf16", "state_output")


# ------------------------------------------------------------ SSD, small
SSD_CASES = [
    # batch, seqlen, H, P, N, G, act, gate, h0, states
    (1, 1, 2, 64, 128, 1, "bf16", True, True, False),
    (2, 5, 3, 64, 128, 1, "f32", True, False, True),
    (1, 63, 2, 64, 128, 1, "bf16", False, True, False),
    (2, 64, 4, 64, 128, 1, "bf16", True, True, False),
    (1, 65, 2, 64, 128, 1, "f32", True, True, True),
    (2, 255, 3, 64, 128, 1, "bf16", True, True, False),
    (1, 256, 2, 64, 128, 1, "bf16", True, False, False),
    (1, 257, 2, 64, 128, 1, "bf16", True, True, False),
    (2, 1000, 4, 64, 128, 2, "bf16", True, True, False),
    (1, 300, 3, 32, 64, 1, "f32", True, True, False),
    (1, 700, 2, 64, 16, 1, "bf16", False, False, False),
    (1, 2100, 2, 64, 128, 1, "bf16", True, True, False),
    (2, 300, 4, 32, 128, 2, "f32", True, True, True),    # token loop, 16 lanes a channel: groups, slices, states
    (1, 150, 2, 64, 100, 1, "bf16", True, True, True),   # 100 of a padded 128, slices, states
    (1, 1100, 2, 128, 64, 1, "bf16", True, True, False), # head_dim 128: the token loop
]


@pytest.mark.parametrize("case", SSD_CASES, ids=lambda c: "b%d_L%d_H%d_P%d_N%d_G%d_%s_g%d_h%d_s%d" % c)
def test_ssd_small(case):
    b, L, H, P, N, G, act, gate, h0, states = case
    say("ssd case", case)
    inp = gen.make_ssd(b, L, H, P, N, G, act=act, seed=L + 3 * H, gate=gate, h0=h0, want_states=states)
    yr, hr, sr = oracle.run_inputs(inp)
    yg, hg, sg = run_ssd(inp)
    check(yg, yr, act, "y")
    check(hg, hr, act, "state_output")
    if states:
        check(sg, sr, act, "states")
        assert np.array_equal(sg[:, -1], hg)


# The chunk kernel cuts each chain (one head of one batch row) into segments of
# whole chunks that any workgroup may take, handing the state over between
# them. Forced cuts: one-chunk segments on a grid far smaller than the items,
# so that items wait on their predecessors and workgroups run several chains.
SEGMENT_CASES = [
    # chunks per segment, workgroups, batch, seqlen, H, G, gate, h0
    (1, 3, 2, 300, 3, 1, True, True),
    (2, 5, 1, 1000, 4, 2, True, False),
    (1, 1, 1, 200, 2, 1, False, True),
    (3, 64, 3, 700, 4, 1, True, True),
]


@pytest.mark.parametrize("case", SEGMENT_CASES, ids=lambda c: "seg%d_wg%d_b%d_L%d_H%d_G%d_g%d_h%d" % c)
def test_ssd_forced_segments(case, monkeypatch):
    sc, wg, b, L, H, G, gate, h0 = case
    say("ssd forced segments", case)
    monkeypatch.setenv("SSCAN_SSD_SEGMENT", "%d,%d" % (sc, wg))
    inp = gen.make_ssd(b, L, H, 64, 128, G, act="bf16", seed=L + 7 * sc + wg, gate=gate, h0=h0)
    yr, hr, _ = oracle.run_inputs(inp)
    yg, hg, _ = run_ssd(inp)
    check(yg, yr, "bf16", "y")
    check(hg, hr, "bf16", "state_output")
    # the cut changes who computes a chunk, not what: the result is bit-identical
    monkeypatch.delenv("SSCAN_SSD_SEGMENT")
    yw, hw, _ = run_ssd(inp)
    assert np.array_equal(yg, yw) and np.array_equal(hg, hw)


def test_ssd_step_chain_equals_oracle():
    inp = gen.make_ssd(2, 12, 3, 64, 128, act="f32", seed=5, gate=True, h0=True)
    yr, hr, _ = oracle.run_inputs(inp)
    x, dt, z = dev(inp.x, "f32"), dev(inp.dt_raw, "f32"), dev(inp.z, "f32")
    B, C = dev(inp.B, "f32"), dev(inp.C, "f32")
    state = par(inp.h0).clone()
    ys = []
    for t in range(inp.seqlen):
        y1, _ = bd.sscan_ssd_step(state, x[:, t:t + 1].contiguous(), dt[:, t:t + 1].contiguous(), par(inp.dt_bias),
                                  par(inp.A_log), B[:, t:t + 1].contiguous(), C[:, t:t + 1].contiguous(),
                                  par(inp.D), z[:, t:t + 1].contiguous(), state_output=state)
        ys.append(host(y1))
    check(np.concatenate(ys, 1), yr, "f32", "y (ssd steps)")
    check(host(state), hr, "f32", "state (ssd steps)")


STEP_CASES = [
    # ssd, batch, seqlen, channels or heads, N, act, gate, bc_eps
    (False, 2, 6, 96, 5, "f32", True, 0.0),     # state_dim below the padded width: entry-wise path
    (False, 3, 5, 64, 8, "bf16", False, 0.0),
    (False, 2, 7, 130, 16, "bf16", True, 1e-6),
    (False, 1, 4, 64, 24, "f32", True, 0.0),
    (False, 2, 5, 64, 64, "bf16", True, 1e-6),
    (False, 1, 3, 32, 40, "f32", False, 0.0),   # 40 of a padded 64
    (True, 2, 6, 3, 16, "bf16", True, 0.0),
    (True, 1, 5, 2, 64, "f32", False, 0.0),
    (True, 2, 4, 2, 128, "bf16", True, 0.0),
    (True, 2, 4, 3, 128, "f32", True, 0.0),
    (False, 2, 4, 64, 128, "bf16", True, 1e-6),
    (False, 1, 3, 32, 100, "f32", False, 0.0),
    (True, 1, 3, 2, 100, "bf16", False, 0.0),  # 100 of a padded 128: entry-wise, 16 lanes a channel
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "ssd%d_b%d_L%d_D%d_N%d_%s_g%d_e%g" % c)
def test_step_chain_shapes(case):
    """One-token calls over a short sequence, the state updated in place, against
    the oracle's scan of the whole sequence."""
    ssd, b, L, D, N, act, gate, eps = case
    say("step case", case)
    if ssd:
        inp = gen.make_ssd(b, L, D, 64, N, act=act, seed=N + L, gate=gate, h0=True)
    else:
        inp = gen.make_mamba1(b, L, D, N, act=act, seed=N + L, gate=gate, h0=True, bc_eps=eps)
    yr, hr, _ = oracle.run_inputs(inp)
    x, dt, B, C = dev(inp.x, act), dev(inp.dt_raw, act), dev(inp.B, act), dev(inp.C, act)
    z = dev(inp.z, act) if gate else None
    state = par(inp.h0).clone()
    ys = []
    for t in range(L):
        one = lambda a: a[:, t:t + 1].clone()  # a fresh (16-byte aligned) allocation
        args = (state, one(x), one(dt), par(inp.dt_bias), par(inp.A_log), one(B), one(C), par(inp.D),
                one(z) if gate else None)
        if ssd:
            y1, _ = bd.sscan_ssd_step(*args, state_output=state)
        else:
            y1, _ = bd.sscan_step(*args, state_output=state, bc_rms_eps=eps)
        ys.append(host(y1))
    check(np.concatenate(ys, 1), yr, act, "y (steps)")
    check(host(state), hr, act, "state (steps)")


@pytest.mark.parametrize("G", [2, 8])
def test_ssd_step_with_groups(G):
    """Mamba-2 decode steps with several B/C groups (Codestral's 8 groups of 16 heads
    at G = 8): head h reads group h // (H / G)."""
    H = 16
    inp = gen.make_ssd(2, 3, H, 64, 128, G, act="bf16", seed=40 + G, gate=True, h0=True)
    say("ssd step groups", G)
    yr, hr, _ = oracle.run_inputs(inp)
    state = par(inp.h0).clone()
    ys = []
    for t in range(inp.seqlen):
        one = lambda a: dev(a[:, t:t + 1], "bf16")
        y1, _ = bd.sscan_ssd_step(state, one(inp.x), one(inp.dt_raw), par(inp.dt_bias), par(inp.A_log), one(inp.B),
                                  one(inp.C), par(inp.D), one(inp.z), state_output=state)
        ys.append(host(y1))
    check(np.concatenate(ys, 1), yr, "bf16", "y (steps)")
    check(host(state), hr, "bf16", "state (steps)")


ATTN_CASES = [
    # batch, seqlen, heads, N, groups, act
    (1, 1, 2, 16, 1, "f32"),
    (2, 37, 4, 16, 2, "f32"),
    (1, 300, 3, 64, 1, "f32"),      # two blocks of keys
    (2, 129, 8, 128, 1, "bf16"),
    (1, 520, 80, 128, 1, "bf16"),   # the 2.7B layer's heads; 17 key tiles, ragged, long gaps
    (1, 200, 128, 64, 8, "bf16"),   # 8 groups of 16 heads in one chunk
    (1, 150, 40, 32, 20, "f32"),    # 2 heads per group: one value per lane, 3 chunks of groups
    (1, 100, 300, 16, 1, "f32"),    # a group wider than a chunk: 128 + 128 + 44 heads
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "b%d_L%d_H%d_N%d_G%d_%s" % c)
def test_ssd_attention_map(case):
    """The hidden attention map against the oracle's, element by element (the map is
    fp32 from inputs that are exact in fp32, so the fp32 bound applies), and the
    map rebuilding the GPU scan's y."""
    b, L, H, N, G, act = case
    say("attention case", case)
    inp = gen.make_ssd(b, L, H, 64, N, G, act=act, seed=L + H, gate=False, h0=False, zero_step_frac=0.02)
    ref = oracle.ssd_attention(inp.dt_raw, inp.dt_bias, inp.A_log, inp.B, inp.C)
    got = host(bd.sscan_ssd_attention(dev(inp.dt_raw, act), par(inp.dt_bias), par(inp.A_log), dev(inp.B, act),
                                      dev(inp.C, act)))
    check(got, ref, "f32", "alpha")
    assert np.all(got[:, np.triu_indices(L, 1)[0], np.triu_indices(L, 1)[1], :] == 0.0)
    yg, _, _ = run_ssd(inp)
    y2 = np.einsum("btsh,bshp->bthp", got, inp.x.astype(np.float64)) + inp.D[None, None, :, None] * inp.x
    check(yg, y2, act, "y from the map")


# ------------------------------------------------------------ invariants and edges
def test_zero_step_on_gpu():
    inp = gen.make_mamba1(2, 40, 128, 16, act="f32", seed=21, gate=True, h0=True, want_states=True)
    inp.dt_raw[:, 7] = -np.inf
    _, _, sg = run_mamba1(inp)
    assert np.array_equal(sg[:, 7], sg[:, 6])
    s = gen.make_ssd(1, 30, 2, 64, 128, act="f32", seed=22, want_states=True)
    s.dt_raw[:, 9] = -np.inf
    _, _, sg = run_ssd(s)
    assert np.array_equal(sg[:, 9], sg[:, 8])


def test_zero_steps_scattered_bf16():
    inp = gen.make_mamba1(2, 2000, 192, 16, act="bf16", seed=23, gate=True, zero_step_frac=0.05)
    yr, hr, _ = oracle.run_inputs(inp)
    yg, hg, _ = run_mamba1(inp)
    check(yg, yr, "bf16", "y")
    check(hg, hr, "bf16", "state_output")


def test_split_sequence_on_gpu():
    inp = gen.make_mamba1(2, 1500, 128, 16, act="f32", seed=24, gate=True, h0=True)
    yw, hw, _ = run_mamba1(inp)
    import copy
    a = copy.copy(inp)
    bpart = copy.copy(inp)
    cut = 700
    for k in ("x", "dt_raw", "z", "B", "C"):
        setattr(a, k, getattr(inp, k)[:, :cut])
        setattr(bpart, k, getattr(inp, k)[:, cut:])
    a.seqlen, bpart.seqlen = cut, inp.seqlen - cut
    ya, ha, _ = run_mamba1(a)
    yb, hb, _ = run_mamba1(bpart, state_input=ha.astype(np.float32))
    yr, hr, _ = oracle.run_inputs(inp)
    check(np.concatenate([ya, yb], 1), yr, "f32", "y (split)")
    check(hb, hr, "f32", "state (split)")
    assert np.max(np.abs(np.concatenate([ya, yb], 1) - yw)) <= 1e-4 * np.max(np.abs(yr))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_wide_decay_rates(act):
    """A from -4e-4 to -36316, the span the Mamba-2 page reports on real weights."""
    inp = gen.make_mamba1(2, 600, 128, 16, act=act, seed=25, gate=True, h0=True, A_log_mode="wide")
    yr, hr, _ = oracle.run_inputs(inp)
    yg, hg, _ = run_mamba1(inp)
    check(yg, yr, act, "y")
    check(hg, hr, act, "state_output")
    s = gen.make_ssd(2, 600, 4, 64, 128, act="bf16", seed=26, A_log_mode="wide")
    yr, hr, _ = oracle.run_inputs(s)
    yg, hg, _ = run_ssd(s)
    check(yg, yr, "bf16", "ssd y")
    check(hg, hr, "bf16", "ssd state")


def test_zero_length_sequence_passes_state_through():
    inp = gen.make_mamba1(2, 0, 64, 16, act="f32", seed=27, h0=True)
    _, hg, _ = run_mamba1(inp)
    assert np.array_equal(hg, inp.h0.astype(np.float64))
    inp = gen.make_mamba1(2, 0, 64, 16, act="f32", seed=27, h0=False)
    _, hg, _ = run_mamba1(inp)
    assert not hg.any()


def test_host_tensors_are_refused():
    inp = gen.make_mamba1(1, 4, 64, 16, act="f32", seed=28)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32))
    with pytest.raises(bd.SscanError) as e:
        bd.sscan_mamba1_fwd(t(inp.x), t(inp.dt_raw), t(inp.dt_bias), t(inp.A_log), t(inp.B), t(inp.C), t(inp.D),
                            y=torch.empty(1, 4, 64), state_output=torch.empty(1, 64, 16))
    assert e.value.name == "SSCAN_ERR_NOT_DEVICE"


def test_decode_steps_replayed_from_a_hip_graph():
    """512-style decode loop captured once and replayed: every replay matches the eager run
    (the kernels launch no memset and allocate nothing)."""
    inp = gen.make_mamba1(4, 24, 256, 16, act="f32", seed=31, gate=True, h0=True)
    x, dt, z = dev(inp.x, "f32"), dev(inp.dt_raw, "f32"), dev(inp.z, "f32")
    B, C = dev(inp.B, "f32"), dev(inp.C, "f32")
    bias, alog, D = par(inp.dt_bias), par(inp.A_log), par(inp.D)
    xs = [x[:, t:t + 1].contiguous() for t in range(inp.seqlen)]
    ds = [dt[:, t:t + 1].contiguous() for t in range(inp.seqlen)]
    zs = [z[:, t:t + 1].contiguous() for t in range(inp.seqlen)]
    Bs = [B[:, t:t + 1].contiguous() for t in range(inp.seqlen)]
    Cs = [C[:, t:t + 1].contiguous() for t in range(inp.seqlen)]
    h0 = par(inp.h0)
    state = h0.clone()
    ys = [torch.empty_like(xs[0]) for _ in range(inp.seqlen)]

    def run():
        for t in range(inp.seqlen):
            bd.sscan_step(state, xs[t], ds[t], bias, alog, Bs[t], Cs[t], D, zs[t], y=ys[t], state_output=state)

    run()
    torch.cuda.synchronize()
    eager_y = torch.cat(ys, 1).clone()
    eager_h = state.clone()
    prev = bd.set_pointer_checks(False)
    g = torch.cuda.CUDAGraph()
    state.copy_(h0)
    with torch.cuda.graph(g):
        run()
    bd.set_pointer_checks(prev)
    for rep in range(3):
        state.copy_(h0)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(ys, 1), eager_y), rep
        assert torch.equal(state, eager_h), rep
    yr, hr, _ = oracle.run_inputs(inp)
    check(host(eager_y), yr, "f32", "y (steps)")
    check(host(eager_h), hr, "f32", "state (steps)")


def test_prompt_entry_points_replayed_from_a_hip_graph():
    """The prompt paths captured together into one HIP graph and replayed three times,
    with eager work between the replays: the SSD chunk kernel (its work queues and the
    flags of segments handing the state on are cleared by a kernel inside the graph),
    the sliced Mamba-1 scan, conv1d + silu, the gated norm and the attention map. Every
    replay must give the eager run's bits."""
    s = gen.make_ssd(1, 2048, 8, 64, 128, act="bf16", seed=61, gate=True, h0=True)
    m = gen.make_mamba1(1, 3000, 64, 16, act="f32", seed=62, gate=True, h0=True)
    sx, sdt, sB, sC, sz = (dev(a, "bf16") for a in (s.x, s.dt_raw, s.B, s.C, s.z))
    mx, mdt, mB, mC, mz = (dev(a, "f32") for a in (m.x, m.dt_raw, m.B, m.C, m.z))
    s_par = [par(a) for a in (s.dt_bias, s.A_log, s.D, s.h0)]
    m_par = [par(a) for a in (m.dt_bias, m.A_log, m.D, m.h0)]
    s_ws = torch.empty(max(bd.sscan_ssd_workspace_size(bd.ssd_desc(sx, sB)), 1), dtype=torch.uint8, device="cuda")
    m_ws = torch.empty(max(bd.sscan_mamba1_workspace_size(bd.mamba1_desc(mx, mB)), 1), dtype=torch.uint8,
                       device="cuda")
    a_ws = torch.empty(1 * 512 * 8 * 12, dtype=torch.uint8, device="cuda")
    sy, sh = torch.empty_like(sx), torch.empty_like(s_par[3])
    my, mh = torch.empty_like(mx), torch.empty_like(m_par[3])
    w = par(np.linspace(-0.5, 0.5, 64 * 4, dtype=np.float32).reshape(64, 4))
    cy, cst = torch.empty_like(mx), torch.empty((1, 64, 3), dtype=torch.float32, device="cuda")
    ny = torch.empty_like(sx.view(1, 2048, 512))
    nw = par(np.linspace(0.5, 1.5, 512, dtype=np.float32))
    alpha = torch.empty((1, 512, 512, 8), dtype=torch.float32, device="cuda")
    sdt5, sB5, sC5 = sdt[:, :512].contiguous(), sB[:, :512].contiguous(), sC[:, :512].contiguous()
    outs = [sy, sh, my, mh, cy, cst, ny, alpha]

    def run():
        bd.sscan_ssd_fwd(sx, sdt, s_par[0], s_par[1], sB, sC, s_par[2], sz, s_par[3], y=sy, state_output=sh,
                         workspace=s_ws)
        bd.sscan_mamba1_fwd(mx, mdt, m_par[0], m_par[1], mB, mC, m_par[2], mz, m_par[3], y=my, state_output=mh,
                            workspace=m_ws)
        bd.sscan_conv1d_silu(mx, w, None, None, out=cy, conv_state_out=cst)
        bd.sscan_gated_rmsnorm(sx.view(1, 2048, 512), sz.view(1, 2048, 512), nw, 1e-5, out=ny)
        bd.sscan_ssd_attention(sdt5, s_par[0], s_par[1], sB5, sC5, alpha=alpha, workspace=a_ws)

    say("graph of the prompt entry points")
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    prev = bd.set_pointer_checks(False)
    g = torch.cuda.CUDAGraph()
    try:
        with torch.cuda.graph(g):
            run()
    finally:
        bd.set_pointer_checks(prev)
    for rep in range(3):
        for o in outs:
            o.fill_(7.0)         # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), (rep, i)
    yr, hr, _ = oracle.run_inputs(s)
    check(host(eager[0]), yr, "bf16", "ssd y")
    check(host(eager[1]), hr, "bf16", "ssd state")
