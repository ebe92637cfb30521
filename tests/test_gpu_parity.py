"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle on
the same seeded inputs. Every case, the five workloads at full size included,
compares every output element; bf16 results are held to the relative L2 budget
and to the element-wise bound of tests/_gpu.py."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from state_space_model_sscan_amd import binding as bd
from state_space_model_sscan_amd import inputs as gen

from _gpu import BF16_RELL2, check, check_all, dev, host, par, rel_l2, run_mamba1, run_ssd, say, ssd_chunk_path

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


@pytest.fixture
def tuning():
    """Set launch-plan overrides for one test; every knob returns to 0 afterwards."""
    set_knobs = []

    def set_knob(knob, value):
        bd.set_tuning(knob, value)
        set_knobs.append(knob)

    yield set_knob
    for k in set_knobs:
        bd.set_tuning(k, 0)




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
    (2, 300, 64, 256, "bf16", True, True, True, 1e-6),     # 256 states: the token loop, 16 lanes of 16
    (1, 2000, 64, 200, "f32", True, True, False, 0.0),     # 200 of a padded 256, several slices
    (3, 77, 40, 129, "f32", False, True, True, 0.0),       # one past 128
]


@pytest.mark.parametrize("case", M1_CASES, ids=lambda c: "b%d_L%d_D%d_N%d_%s_g%d_h%d_s%d_e%g" % c)
def test_mamba1_small(case):
    b, L, Dc, N, act, gate, h0, states, eps = case
    say("mamba1 case", case)
    inp = gen.make_mamba1(b, L, Dc, N, act=act, seed=L * 7 + Dc, gate=gate, h0=h0, bc_eps=eps,
                          want_states=states)
    check_all(inp, run_mamba1(inp), oracle.run_inputs(inp), "mamba1", states=states)


# The plan gives state_dim 16/32/64 to the quad-lane kernel on wide shapes and to the
# row-per-channel kernel on the others; these cases force the kernel through the
# lanes-per-channel override: 4 selects the quad-lane kernel (state_dim 16/32/64,
# channels in whole 16-byte pieces), 1 and 2 the general kernel.
LANE_CASES = [
    # lanes, batch, seqlen, channels, N, act, gate, h0, states, bc_eps
    (1, 2, 300, 256, 16, "bf16", True, True, False, 1e-6),
    (2, 3, 129, 192, 32, "f32", True, False, True, 0.0),
    (4, 2, 1000, 128, 16, "f32", False, True, False, 0.0),
    (4, 1, 77, 64, 64, "bf16", True, True, True, 1e-5),
    (4, 3, 300, 136, 16, "bf16", True, True, True, 1e-6),   # a part-filled block of 64 channels
    (4, 1, 3000, 64, 32, "f32", True, True, False, 0.0),    # several slices
    (4, 2, 257, 200, 64, "bf16", False, False, True, 0.0),  # ragged tile, per-token states
]


@pytest.mark.parametrize("case", LANE_CASES, ids=lambda c: "K%d_b%d_L%d_D%d_N%d_%s_g%d_h%d_s%d_e%g" % c)
def test_mamba1_forced_lanes(case, tuning):
    K, b, L, Dc, N, act, gate, h0, states, eps = case
    say("mamba1 forced lanes", case)
    tuning(bd.TUNE_M1_LANES, K)
    inp = gen.make_mamba1(b, L, Dc, N, act=act, seed=L * 5 + Dc + K, gate=gate, h0=h0, bc_eps=eps,
                          want_states=states)
    check_all(inp, run_mamba1(inp), oracle.run_inputs(inp), "mamba1", states=states)


def test_mamba1_grouped_B_C():
    inp = gen.make_mamba1(2, 300, 256, 16, ngroups=2, act="f32", seed=11, gate=True, h0=True)
    check_all(inp, run_mamba1(inp), oracle.run_inputs(inp), "mamba1")


# ------------------------------------------------------------ the five workloads, every element
def test_workload0_full():
    inp = gen.make_workload(0)
    say("workload 0", gen.WORKLOADS[0]["name"])
    check_all(inp, run_mamba1(inp), oracle.run_inputs(inp), "mamba1", states=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", [1, 3])
def test_mamba1_workload_full_size(wid):
    """Workloads 1 (Mamba-130m layer) and 3 (Falcon-Mamba-7b width) at full size, every element."""
    inp = gen.make_workload(wid)
    say("workload", wid, gen.WORKLOADS[wid]["name"])
    got = run_mamba1(inp)
    say("  oracle")
    check_all(inp, got, oracle.run_inputs(inp), "mamba1")


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


@pytest.mark.timeout(900)
def test_workload4_ssd_full_size():
    """The Mamba-2 2.7B layer at full size, every element (the give-up word read back as 0)."""
    inp = gen.make_workload(4)
    say("workload 4", gen.WORKLOADS[4]["name"])
    got = run_ssd(inp)
    say("  oracle")
    check_all(inp, got, oracle.run_inputs(inp), "ssd")


SPLIT_CASES = [
    # two passes (the plan's, 0) or one pass (1), chunks per segment, batch, seqlen, H, G, h0
    (0, 0, 1, 8192, 8, 1, True),     # few chains: two passes
    (1, 0, 2, 1000, 6, 2, True),     # one pass, whole chains
    (1, 2, 2, 700, 4, 1, False),     # one pass, segments of two chunks handing their states on
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "tp%d_seg%d_b%d_L%d_H%d_G%d_h%d" % c)
def test_ssd_split_state_parity(case, tuning):
    """The precise form of the bf16 chunk path (state and w x as two bf16 parts each)
    against the oracle, in one pass and in two."""
    tp, seg, b, L, H, G, h0 = case
    say("ssd split state", case)
    tuning(bd.TUNE_SSD_SPLIT_STATE, 1)
    if tp:
        tuning(bd.TUNE_SSD_TWO_PASS, tp)
    if seg:
        tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, seg)
    inp = gen.make_ssd(b, L, H, 64, 128, G, act="bf16", seed=L + H, gate=True, h0=h0)
    check_all(inp, run_ssd(inp), oracle.run_inputs(inp), "ssd")


@pytest.mark.parametrize("split", [0, 1])
def test_ssd_long_memory_65536_tokens(split, tuning):
    """The long-memory heads over 65,536 tokens, in both forms of the bf16 chunk path: the
    roundings are relative to the terms they round, so the error does not grow with the
    length (measured: the same as at 8192 tokens)."""
    inp = gen.make_ssd(1, 65536, 8, 64, 128, act="bf16", seed=81, gate=True, h0=True)
    inp.A_log = np.log(np.geomspace(4e-4, 1e-2, 8)).astype(np.float32)
    tuning(bd.TUNE_SSD_SPLIT_STATE, split)
    say("ssd long memory, 65536 tokens, precise form" if split else "ssd long memory, 65536 tokens")
    check_all(inp, run_ssd(inp), oracle.run_inputs(inp), "ssd")


def test_ssd_split_state_long_memory(tuning):
    """With slow decays the state sums thousands of tokens and its bf16 rounding as C reads
    it, with that of w x, sets y's error. The precise form keeps both to about 16
    significant bits: y and the final state come out closer to the oracle than on the
    default form, within half the bf16 budget."""
    inp = gen.make_ssd(1, 8192, 8, 64, 128, act="bf16", seed=81, gate=True, h0=True)
    inp.A_log = np.log(np.geomspace(4e-4, 1e-2, 8)).astype(np.float32)
    ref = oracle.run_inputs(inp)
    fast = run_ssd(inp)
    tuning(bd.TUNE_SSD_SPLIT_STATE, 1)
    precise = run_ssd(inp)
    check_all(inp, precise, ref, "ssd")
    e_fast = [rel_l2(fast[i], ref[i]) for i in (0, 1)]
    e_precise = [rel_l2(precise[i], ref[i]) for i in (0, 1)]
    say("  rel_l2 y, state: default %.3e %.3e, precise %.3e %.3e" % (*e_fast, *e_precise))
    assert e_precise[0] < e_fast[0] and e_precise[1] < e_fast[1]
    assert max(e_precise) <= BF16_RELL2 / 2


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_ssd_long_memory(act):
    """8192 tokens on the chunk kernels with decays near the slowest the Mamba-2 page reports
    on real weights (|A| from 4e-4 to 1e-2): the state sums thousands of tokens, the case
    where the bf16 operands of w*x and of the state as C reads it would accumulate error
    (and, for fp32 activations, where the fp32 chunk kernel's sums run longest)."""
    inp = gen.make_ssd(1, 8192, 8, 64, 128, act=act, seed=81, gate=True, h0=True)
    inp.A_log = np.log(np.geomspace(4e-4, 1e-2, 8)).astype(np.float32)
    say("ssd long memory: A", -np.exp(inp.A_log.astype(np.float64)))
    got = run_ssd(inp)
    check_all(inp, got, oracle.run_inputs(inp), "ssd")


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_ssd_codestral_heads_and_groups(act):
    """Codestral's layout on the chunk kernels: 128 heads in 8 groups of B and C."""
    inp = gen.make_ssd(1, 1000, 128, 64, 128, 8, act=act, seed=82, gate=True, h0=True)
    check_all(inp, run_ssd(inp), oracle.run_inputs(inp), "ssd")


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
    (1, 300, 3, 32, 64, 1, "f32", True, True, False),    # head_dim 32: the token loop
    (1, 700, 2, 64, 16, 1, "bf16", False, False, False), # state_dim 16: the token loop
    (1, 2100, 2, 64, 128, 1, "bf16", True, True, False),
    (2, 300, 4, 32, 128, 2, "f32", True, True, True),    # token loop, 16 lanes a channel: groups, slices, states
    (1, 150, 2, 64, 100, 1, "bf16", True, True, True),   # 100 of a padded 128, slices, states
    (1, 1100, 2, 128, 64, 1, "bf16", True, True, False), # head_dim 128, state_dim 64 (padded): chunk kernel
    # head_dim and state_dim 128: bf16 with states and groups on the token loop, with
    # slices; head_dim 160 (not 64 times a power of two) and 96 on the token loop
    (1, 500, 2, 128, 128, 2, "bf16", True, True, True),
    (1, 300, 2, 160, 64, 1, "f32", True, False, False),
    (1, 400, 3, 96, 128, 1, "bf16", True, True, False),
    # head_dim 128 and 256 on the chunk kernels (each head as 64-column heads that
    # share its step, decay and D): chunk edges, ragged tails, groups
    (1, 600, 2, 128, 128, 1, "f32", True, True, False),
    (2, 700, 3, 128, 128, 1, "bf16", True, True, False),
    (1, 129, 4, 128, 128, 2, "bf16", False, False, False),
    (2, 300, 4, 128, 128, 4, "f32", True, False, False),
    (1, 1500, 2, 256, 128, 2, "bf16", True, True, False),
    (1, 65, 2, 256, 128, 1, "f32", True, True, False),
    # state_dim 64..127 on the chunk kernels (B, C and the states zero-padded to 128 in
    # the workspace); state_dim 64 with per-token states on the token loop
    (2, 500, 3, 64, 64, 1, "bf16", True, True, False),
    (2, 65, 2, 64, 64, 1, "f32", True, False, False),
    (1, 257, 2, 64, 100, 2, "f32", True, True, False),
    (1, 777, 4, 64, 80, 1, "bf16", False, True, False),
    (1, 600, 2, 64, 64, 1, "bf16", True, True, True),
    # fp32 activations on the fp32 MFMA chunk kernel: one token, chunk edges, ragged
    # tails, groups, long sequences (segments)
    (1, 1, 2, 64, 128, 1, "f32", True, True, False),
    (2, 63, 3, 64, 128, 1, "f32", False, True, False),
    (1, 64, 2, 64, 128, 1, "f32", True, False, False),
    (2, 257, 4, 64, 128, 2, "f32", True, True, False),
    (1, 1000, 4, 64, 128, 4, "f32", True, False, False),
    (1, 2100, 2, 64, 128, 1, "f32", True, True, False),
]


@pytest.mark.parametrize("case", SSD_CASES, ids=lambda c: "b%d_L%d_H%d_P%d_N%d_G%d_%s_g%d_h%d_s%d" % c)
def test_ssd_small(case):
    b, L, H, P, N, G, act, gate, h0, states = case
    say("ssd case", case)
    inp = gen.make_ssd(b, L, H, P, N, G, act=act, seed=L + 3 * H, gate=gate, h0=h0, want_states=states)
    path = "ssd" if ssd_chunk_path(inp, states) else "mamba1"  # the token loop computes in fp32
    check_all(inp, run_ssd(inp), oracle.run_inputs(inp), path, states=states)


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
def test_ssd_forced_segments(case, tuning):
    sc, wg, b, L, H, G, gate, h0 = case
    say("ssd forced segments", case)
    tuning(bd.TUNE_SSD_TWO_PASS, 1)  # one pass: the hand-offs between segments
    tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, sc)
    tuning(bd.TUNE_SSD_WORKGROUPS, wg)
    inp = gen.make_ssd(b, L, H, 64, 128, G, act="bf16", seed=L + 7 * sc + wg, gate=gate, h0=h0)
    got = run_ssd(inp)
    check_all(inp, got, oracle.run_inputs(inp), "ssd")
    # the cut changes who computes a chunk, not what: the result is bit-identical
    bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 0)
    bd.set_tuning(bd.TUNE_SSD_WORKGROUPS, 0)
    yw, hw, _ = run_ssd(inp)
    assert np.array_equal(got[0], yw) and np.array_equal(got[1], hw)


F32_SEGMENT_CASES = [
    # chunks per segment, workgroups, batch, seqlen, H, G, gate, h0
    (1, 3, 2, 300, 3, 1, True, True),
    (3, 64, 3, 700, 4, 2, True, True),
]


@pytest.mark.parametrize("case", F32_SEGMENT_CASES, ids=lambda c: "seg%d_wg%d_b%d_L%d_H%d_G%d_g%d_h%d" % c)
def test_ssd_f32_forced_segments(case, tuning):
    """The fp32 chunk kernel's hand-offs: forced one- and three-chunk segments on small
    grids, against the oracle and bit-identical to the library's own cut."""
    sc, wg, b, L, H, G, gate, h0 = case
    say("ssd f32 forced segments", case)
    tuning(bd.TUNE_SSD_TWO_PASS, 1)
    tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, sc)
    tuning(bd.TUNE_SSD_WORKGROUPS, wg)
    inp = gen.make_ssd(b, L, H, 64, 128, G, act="f32", seed=L + 7 * sc + wg, gate=gate, h0=h0)
    got = run_ssd(inp)
    check_all(inp, got, oracle.run_inputs(inp), "ssd")
    bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 0)
    bd.set_tuning(bd.TUNE_SSD_WORKGROUPS, 0)
    yw, hw, _ = run_ssd(inp)
    assert np.array_equal(got[0], yw) and np.array_equal(got[1], hw)


def _as_64_column_heads(inp):
    """The same problem with each head of 64 m columns written as m heads of 64 columns,
    each with its head's step, decay and D: x, z, y and the states keep their bytes."""
    m = inp.head_dim // 64
    rep = lambda a: None if a is None else np.ascontiguousarray(np.repeat(a, m, axis=-1))
    b, L, H = inp.batch, inp.seqlen, inp.nheads
    cols = lambda a: None if a is None else np.ascontiguousarray(a.reshape(b, L, H * m, 64))
    return dataclasses.replace(
        inp, nheads=H * m, head_dim=64, x=cols(inp.x), z=cols(inp.z), dt_raw=rep(inp.dt_raw),
        dt_bias=rep(inp.dt_bias), A_log=rep(inp.A_log), D=rep(inp.D),
        h0=None if inp.h0 is None else np.ascontiguousarray(inp.h0.reshape(b, H * m, 64, inp.state_dim)))


HEAD_DIM_CASES = [
    # head_dim, batch, seqlen, H, G, act, gate, h0, segment chunks (0: the plan's)
    (128, 2, 700, 3, 1, "bf16", True, True, 0),
    (128, 1, 1000, 4, 2, "bf16", True, False, 3),
    (256, 1, 500, 2, 1, "bf16", False, True, 1),
    (128, 2, 300, 4, 2, "f32", True, True, 0),
    (256, 1, 600, 2, 2, "f32", True, True, 2),
]


@pytest.mark.parametrize("case", HEAD_DIM_CASES, ids=lambda c: "P%d_b%d_L%d_H%d_G%d_%s_g%d_h%d_seg%d" % c)
def test_ssd_wide_heads_equal_their_64_column_heads(case, tuning):
    """The chunk kernels take a head of 64 m columns as m heads of 64 columns that share
    its step, decay and D. Written out that way by the caller (dt_raw, dt_bias, A_log and
    D repeated per column block), the same call must give bit-identical y and state;
    both against the oracle."""
    P, b, L, H, G, act, gate, h0, seg = case
    say("ssd wide heads", case)
    if seg:
        tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, seg)
    inp = gen.make_ssd(b, L, H, P, 128, G, act=act, seed=P + L + H, gate=gate, h0=h0)
    assert ssd_chunk_path(inp, False)
    wide = run_ssd(inp)
    narrow = run_ssd(_as_64_column_heads(inp))
    assert np.array_equal(wide[0].reshape(-1), narrow[0].reshape(-1))
    assert np.array_equal(wide[1].reshape(-1), narrow[1].reshape(-1))
    check_all(inp, wide, oracle.run_inputs(inp), "ssd")


NARROW_STATE_CASES = [
    # state_dim, head_dim, batch, seqlen, H, G, act, h0, segment chunks (0: the plan's)
    (64, 64, 2, 700, 3, 1, "bf16", True, 0),
    (64, 128, 1, 900, 2, 2, "bf16", True, 3),
    (96, 64, 1, 500, 4, 1, "f32", True, 1),
    (64, 64, 2, 300, 2, 2, "f32", False, 0),
]


@pytest.mark.parametrize("case", NARROW_STATE_CASES, ids=lambda c: "N%d_P%d_b%d_L%d_H%d_G%d_%s_h%d_seg%d" % c)
def test_ssd_narrow_state_equals_zero_padded(case, tuning):
    """state_dim below 128 on the chunk kernels: the library pads B, C and the entering
    state with zero states. The caller padding them itself must give bit-identical y and
    the same state, whose padded entries come out exactly zero; both against the oracle."""
    N, P, b, L, H, G, act, h0, seg = case
    say("ssd narrow state", case)
    if seg:
        tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, seg)
    inp = gen.make_ssd(b, L, H, P, N, G, act=act, seed=N + P + L, gate=True, h0=h0)
    assert ssd_chunk_path(inp, False)
    pad = lambda a: None if a is None else np.ascontiguousarray(
        np.concatenate([a, np.zeros(a.shape[:-1] + (128 - N,), a.dtype)], axis=-1))
    wide = dataclasses.replace(inp, state_dim=128, B=pad(inp.B), C=pad(inp.C), h0=pad(inp.h0))
    got = run_ssd(inp)
    ref = run_ssd(wide)
    assert np.array_equal(got[0], ref[0])
    assert np.array_equal(got[1], ref[1][..., :N])
    assert not np.any(ref[1][..., N:])
    check_all(inp, got, oracle.run_inputs(inp), "ssd")


TWO_PASS_CASES = [
    # chunks per segment (0: the plan's), workgroups (0: the plan's), batch, seqlen, H, P, N, G, act, h0
    (1, 0, 1, 300, 2, 64, 128, 1, "bf16", True),
    (0, 0, 1, 1, 2, 64, 128, 1, "bf16", True),    # one chunk: the second pass alone
    (0, 0, 2, 5000, 6, 64, 128, 2, "bf16", True), # the plan's cut and grid
    (3, 5, 2, 1000, 4, 64, 128, 2, "bf16", False),
    (0, 0, 1, 4000, 2, 64, 128, 1, "bf16", True),
    (2, 0, 1, 700, 2, 128, 128, 1, "bf16", True),
    (2, 3, 1, 600, 3, 64, 64, 1, "bf16", True),
    (1, 0, 2, 257, 2, 64, 128, 1, "f32", True),
    (4, 7, 1, 1500, 4, 64, 128, 2, "f32", False),
    (0, 0, 1, 3000, 2, 128, 128, 1, "f32", True),
    (3, 0, 1, 900, 2, 64, 96, 1, "f32", True),
]


@pytest.mark.parametrize("case", TWO_PASS_CASES, ids=lambda c: "seg%d_wg%d_b%d_L%d_H%d_P%d_N%d_G%d_%s_h%d" % c)
def test_ssd_two_pass(case, tuning):
    """The chunk path in two passes: every segment but the last scanned from a zero state
    (its state and decay sum kept), then every segment from its entering state folded
    from those. Against the oracle; fp32 also against the one-pass form at the fp32
    bound (the fold rounds differently, so the two are close, not identical)."""
    sc, wg, b, L, H, P, N, G, act, h0 = case
    say("ssd two passes", case)
    inp = gen.make_ssd(b, L, H, P, N, G, act=act, seed=L + H + P + N, gate=True, h0=h0)
    assert ssd_chunk_path(inp, False)
    tuning(bd.TUNE_SSD_TWO_PASS, 2)
    if sc:
        tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, sc)
    if wg:
        tuning(bd.TUNE_SSD_WORKGROUPS, wg)
    two = run_ssd(inp)
    check_all(inp, two, oracle.run_inputs(inp), "ssd")
    bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 1)
    one = run_ssd(inp)
    if act == "f32":
        check(two[0], one[0], "f32", "y (two passes vs one)")
        check(two[1], one[1], "f32", "state (two passes vs one)")


def test_ssd_f32_chunk_kernel_agrees_with_token_loop():
    """fp32 activations: the fp32 MFMA chunk kernel and the token loop restate the same
    recurrence in fp32, so both meet the oracle and each other at the fp32 bound."""
    inp = gen.make_ssd(2, 900, 4, 64, 128, 2, act="f32", seed=321, gate=True, h0=True)
    ref = oracle.run_inputs(inp)
    chunk = run_ssd(inp)
    loop = run_ssd(inp, token_loop=True)
    check_all(inp, chunk, ref, "ssd")
    check_all(inp, loop, ref, "mamba1")
    check(chunk[0], loop[0], "f32", "y (chunk vs token loop)")
    check(chunk[1], loop[1], "f32", "state (chunk vs token loop)")


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_ssd_handoff_give_up_poisons_dependent_outputs(tuning, act):
    """A state hand-off wait that gives up (forced from the host: the give-up word is raised
    before the kernel starts, so every wait ends at once) must not leave wrong numbers
    behind: the first segment of every head is exact, everything after it is NaN, and the
    word reads back nonzero. No wait blocks and no kernel faults. Both chunk kernels."""
    inp = gen.make_ssd(2, 700, 4, 64, 128, act=act, seed=83, gate=True, h0=True)
    tuning(bd.TUNE_SSD_TWO_PASS, 1)            # one pass: segments hand their states on in turn
    tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 2)      # segments of 128 tokens
    good_y, good_h, _ = run_ssd(inp)
    tuning(bd.TUNE_SSD_GIVE_UP, 1)
    bad_y, bad_h, _ = run_ssd(inp, expect_giveup=True)
    assert np.array_equal(bad_y[:, :128], good_y[:, :128])
    assert np.all(np.isnan(bad_y[:, 128:]))
    assert np.all(np.isnan(bad_h))
    bd.set_tuning(bd.TUNE_SSD_GIVE_UP, 0)
    again_y, _, _ = run_ssd(inp)
    assert np.array_equal(again_y, good_y)


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
    (False, 2, 4, 64, 256, "bf16", True, 1e-6),  # 256 states
    (False, 1, 3, 32, 150, "f32", False, 0.0),   # 150 of a padded 256: entry-wise
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
    check_all(inp, (np.concatenate(ys, 1), host(state)), (yr, hr), "mamba1")


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
    check_all(inp, (np.concatenate(ys, 1), host(state)), (yr, hr), "mamba1")


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
    check_all(inp, run_mamba1(inp), oracle.run_inputs(inp), "mamba1")


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
    check_all(inp, run_mamba1(inp), oracle.run_inputs(inp), "mamba1")
    s = gen.make_ssd(2, 600, 4, 64, 128, act=act, seed=26, A_log_mode="wide")
    check_all(s, run_ssd(s), oracle.run_inputs(s), "ssd")


def test_zero_length_sequence_passes_state_through():
    inp = gen.make_mamba1(2, 0, 64, 16, act="f32", seed=27, h0=True)
    _, hg, _ = run_mamba1(inp)
    assert np.array_equal(hg, inp.h0.astype(np.float64))
    inp = gen.make_mamba1(2, 0, 64, 16, act="f32", seed=27, h0=False)
    _, hg, _ = run_mamba1(inp)
    assert not hg.any()


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_ssd_zero_length_sequence_passes_state_through(act):
    """seqlen 0 at the chunk kernels' shape (head_dim 64, state_dim 128): the state passes
    through unchanged (zeros without an entering state) and y is empty."""
    for h0 in (True, False):
        inp = gen.make_ssd(2, 0, 3, 64, 128, act=act, seed=29, gate=True, h0=h0)
        y, hg, _ = run_ssd(inp)
        assert y.size == 0
        if h0:
            assert np.array_equal(hg, inp.h0.astype(np.float64))
        else:
            assert not hg.any()


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_batch_zero_calls_are_no_ops(act):
    """batch 0 (every tensor empty) through every entry point: each call succeeds and
    launches nothing that reads or writes (the outputs have no elements)."""
    m = gen.make_mamba1(0, 7, 64, 16, act=act, seed=30, gate=True, h0=True)
    x, dt, z, B, C = (dev(a, act) for a in (m.x, m.dt_raw, m.z, m.B, m.C))
    y, h, _ = bd.sscan_mamba1_fwd(x, dt, par(m.dt_bias), par(m.A_log), B, C, par(m.D), z, par(m.h0))
    assert y.numel() == 0 and h.numel() == 0
    one = lambda t: t[:, :1].contiguous()
    y, h = bd.sscan_step(par(m.h0), one(x), one(dt), par(m.dt_bias), par(m.A_log), one(B), one(C), par(m.D), one(z))
    assert y.numel() == 0 and h.numel() == 0
    s = gen.make_ssd(0, 70, 4, 64, 128, act=act, seed=30, gate=True, h0=True)
    x, dt, z, B, C = (dev(a, act) for a in (s.x, s.dt_raw, s.z, s.B, s.C))
    for fwd in (bd.sscan_ssd_fwd, bd.sscan_ssd_fwd_noalloc):
        y, h, _ = fwd(x, dt, par(s.dt_bias), par(s.A_log), B, C, par(s.D), z, par(s.h0))
        assert y.numel() == 0 and h.numel() == 0
    y, h = bd.sscan_ssd_step(par(s.h0), one(x), one(dt), par(s.dt_bias), par(s.A_log), one(B), one(C),
                             par(s.D), one(z))
    assert y.numel() == 0 and h.numel() == 0
    alpha = bd.sscan_ssd_attention(dt, par(s.dt_bias), par(s.A_log), B, C)
    assert alpha.numel() == 0
    w = torch.ones(64, 4, device="cuda")
    out, st = bd.sscan_conv1d_silu(dev(m.x, act), w, conv_state_out=torch.empty(0, 64, 3, device="cuda"))
    assert out.numel() == 0 and st.numel() == 0
    out = bd.sscan_gated_rmsnorm(dev(m.x, act), dev(m.z, act), torch.ones(64, device="cuda"), 1e-5)
    assert out.numel() == 0
    torch.cuda.synchronize()


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
    check_all(s, (host(eager[0]), host(eager[1])), oracle.run_inputs(s), "ssd")


HPW_CASES = [
    # batch, seqlen, H, G, gate, h0, segment chunks (0: the plan's)
    (2, 1000, 8, 1, True, True, 0),
    (1, 777, 16, 8, True, False, 3),    # two heads per group: pairs never straddle groups
    (2, 300, 6, 3, False, True, 1),
]


@pytest.mark.parametrize("case", HPW_CASES, ids=lambda c: "b%d_L%d_H%d_G%d_g%d_h%d_seg%d" % c)
def test_ssd_two_heads_per_workgroup_equals_one(case, tuning):
    """The chunk kernel with two heads per workgroup (shared B, C and C B^T tiles) against
    the same kernel with one head per workgroup: each head's arithmetic is the same, so the
    results are bit-identical; both against the oracle."""
    b, L, H, G, gate, h0, seg = case
    say("ssd heads per workgroup", case)
    tuning(bd.TUNE_SSD_TWO_PASS, 1)  # (two heads per workgroup run in one pass only)
    if seg:
        tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, seg)
    inp = gen.make_ssd(b, L, H, 64, 128, G, act="bf16", seed=L + H + G, gate=gate, h0=h0)
    one = run_ssd(inp)
    tuning(bd.TUNE_SSD_HEADS_PER_WORKGROUP, 2)
    two = run_ssd(inp)
    assert np.array_equal(two[0], one[0]) and np.array_equal(two[1], one[1])
    check_all(inp, two, oracle.run_inputs(inp), "ssd")
