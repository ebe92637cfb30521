"""A seeded sweep of random problem shapes through both scans, every output element
against the oracle with the same bounds as the other parity tests.

The shapes are drawn so that the launch plans pick each of their kernels: for
Mamba-1 the row, quad and general prompt kernels and the token loop (state_dim up to
256, groups, the B/C norm, slices of long sequences), for the SSD the MFMA chunk
kernels (bf16 and fp32, head_dim 64 or 128, state_dim 64 to 128, with segments) and the
token loop (other head and state sizes, per-token states). Lengths include 1, chunk and tile
edges and ragged tails; some cases drop 5% of the tokens to a zero step (dt_raw = -inf) and
some SSD cases draw A over the pages' whole span (ln 4e-4 .. ln 36316), and some bf16 SSD cases
take the chunk path's precise form. Sizes stay small enough for the oracle to take well under a
second per case."""
import numpy as np
import pytest
import torch

import oracle
from state_space_model_sscan_amd import binding as bd
from state_space_model_sscan_amd import inputs as gen

from _gpu import check_all, run_mamba1, run_ssd, say, ssd_chunk_path

pytestmark = pytest.mark.gpu

UPDATES_MAX = 40_000_000  # batch x tokens x channels x state_dim per case


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def _mamba1_cases(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        N = int(rng.choice([1, 3, 8, 16, 16, 16, 24, 32, 33, 64, 100, 128, 129, 256]))
        G = int(rng.choice([1, 1, 1, 2, 4]))
        # log-uniform widths, so that narrow problems with long (sliced) sequences come up
        Dc = G * 64 * int(rng.integers(1, 4)) if G > 1 else int(np.exp(rng.uniform(0.0, np.log(1200.0))))
        b = int(rng.integers(1, 5))
        L = int(rng.choice([1, 2, 15, 16, 63, 64, 65, 127, 128, 129, 300, 777, 2049]))
        if b * L * Dc * N > UPDATES_MAX:
            continue
        act = str(rng.choice(["f32", "bf16"]))
        cases.append(dict(batch=b, seqlen=L, channels=Dc, state_dim=N, ngroups=G, act=act,
                          gate=bool(rng.random() < 0.7), h0=bool(rng.random() < 0.5),
                          bc_eps=float(rng.choice([0.0, 0.0, 1e-6, 1e-3])),
                          want_states=bool(rng.random() < 0.25 and b * L * Dc * N < 4_000_000),
                          zero_step_frac=float(rng.choice([0.0, 0.0, 0.0, 0.05])),
                          seed=int(rng.integers(1 << 30))))
    return cases


def _ssd_cases(n=32, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        if rng.random() < 0.5:  # the MFMA chunk kernels' shapes (bf16, and fp32 a third of the time)
            P, N = int(rng.choice([64, 64, 128])), int(rng.choice([128, 128, 64]))
            act, states = str(rng.choice(["bf16", "bf16", "f32"])), False
        else:
            P = int(rng.choice([1, 2, 16, 32, 64, 64, 96, 128]))
            N = int(rng.choice([1, 5, 16, 32, 64, 100, 128]))
            act = str(rng.choice(["f32", "bf16"]))
            states = bool(rng.random() < 0.3)
        G = int(rng.choice([1, 1, 2, 4]))
        hpg = int(rng.integers(1, 5))
        if G > 1 and (hpg * P) % 64 != 0:
            continue
        H = G * hpg
        b = int(rng.integers(1, 4))
        L = int(rng.choice([1, 2, 63, 64, 65, 255, 256, 257, 700, 1500, 3000]))
        upd = b * L * H * P * N
        if upd > UPDATES_MAX or (states and upd > 4_000_000):
            continue
        cases.append(dict(batch=b, seqlen=L, nheads=H, head_dim=P, state_dim=N, ngroups=G, act=act,
                          gate=bool(rng.random() < 0.7), h0=bool(rng.random() < 0.5), want_states=states,
                          zero_step_frac=float(rng.choice([0.0, 0.0, 0.0, 0.05])),
                          A_log_mode=str(rng.choice(["random", "random", "random", "wide"])),
                          split=bool(act == "bf16" and rng.random() < 0.3),
                          seed=int(rng.integers(1 << 30))))
    return cases


def _id(c):
    return "_".join("%s%s" % (k[:2], v) for k, v in c.items() if k != "seed")


@pytest.mark.parametrize("case", _mamba1_cases(), ids=_id)
def test_mamba1_random_shape(case):
    say("mamba1 random", case)
    c = dict(case)
    inp = gen.make_mamba1(c.pop("batch"), c.pop("seqlen"), c.pop("channels"), A_log_mode="random", **c)
    check_all(inp, run_mamba1(inp), oracle.run_inputs(inp), "mamba1", states=inp.want_states)


@pytest.mark.parametrize("case", _ssd_cases(), ids=_id)
def test_ssd_random_shape(case):
    say("ssd random", case)
    c = dict(case)
    split = c.pop("split")  # bf16: the chunk path's precise form (state and w x in two parts)
    inp = gen.make_ssd(c.pop("batch"), c.pop("seqlen"), c.pop("nheads"), c.pop("head_dim"), c.pop("state_dim"),
                       c.pop("ngroups"), **c)
    path = "ssd" if ssd_chunk_path(inp, inp.want_states) else "mamba1"  # the token loop computes in fp32
    prev = bd.set_tuning(bd.TUNE_SSD_SPLIT_STATE, 1 if split else 0)
    try:
        got = run_ssd(inp)
    finally:
        bd.set_tuning(bd.TUNE_SSD_SPLIT_STATE, prev)
    check_all(inp, got, oracle.run_inputs(inp), path, states=inp.want_states)
