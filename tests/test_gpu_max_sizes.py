"""Parity at the largest batch rows the fast kernels take, and just past them.

The prompt kernels address a batch row of x, dt_raw, z and y (and of B and C) with
32-bit buffer offsets, so the library sends a row of 2^31 bytes or more to the
token-loop kernels, which index in 64 bits. These tests run one shape a token below
that boundary (the fast kernel, with two batch rows, so that every tensor spans
more than 2^32 bytes) and one a token past it (the token loop), for the Mamba-1 scan
and for the SSD. The oracle computes a sample of whole channels (Mamba-1) or whole
heads (SSD) over the full length: channels and heads are independent given B and C,
which every channel shares ("Mamba", nnterp guide, section "The values"; "Mamba-2",
section "The mixer's values"). Those outputs are compared element by element under
the same bounds as every other parity test.
"""
import copy

import numpy as np
import pytest
import torch

import oracle
from state_space_model_sscan_amd import binding as bd
from state_space_model_sscan_amd import inputs as gen

from _gpu import check_all, dev, par, say

pytestmark = pytest.mark.gpu

ROW_LIMIT = 1 << 31  # bytes of one batch row that the fast kernels' offsets can span


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def _cols(a, idx, axis):
    return None if a is None else np.ascontiguousarray(np.take(a, idx, axis=axis))


def _mamba1_subset(inp, chans):
    """The same problem restricted to some channels (one group of B and C: unchanged)."""
    s = copy.copy(inp)
    s.channels = len(chans)
    s.x, s.dt_raw, s.z = _cols(inp.x, chans, 2), _cols(inp.dt_raw, chans, 2), _cols(inp.z, chans, 2)
    s.dt_bias, s.A_log, s.D = _cols(inp.dt_bias, chans, 0), _cols(inp.A_log, chans, 0), _cols(inp.D, chans, 0)
    s.h0 = _cols(inp.h0, chans, 1)
    return s


def _ssd_subset(inp, heads):
    s = copy.copy(inp)
    s.nheads = len(heads)
    s.x, s.dt_raw, s.z = _cols(inp.x, heads, 2), _cols(inp.dt_raw, heads, 2), _cols(inp.z, heads, 2)
    s.dt_bias, s.A_log, s.D = _cols(inp.dt_bias, heads, 0), _cols(inp.A_log, heads, 0), _cols(inp.D, heads, 0)
    s.h0 = _cols(inp.h0, heads, 1)
    return s


def _pick(t, idx, axis):
    """Outputs at the sampled channels or heads, from the GPU as float64."""
    ix = torch.as_tensor(idx, device=t.device)
    return t.index_select(axis, ix).float().cpu().numpy().astype(np.float64)


# batch, seqlen, channels: one token below and one past a 2^31-byte batch row of bf16
M1_MAX = [(2, ROW_LIMIT // (1536 * 2) - 0, 1536), (1, ROW_LIMIT // (1536 * 2) + 1, 1536)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", M1_MAX, ids=lambda c: "b%d_L%d_D%d" % c)
def test_mamba1_largest_rows(case):
    b, L, Dc = case
    below = L * Dc * 2 < ROW_LIMIT
    say("mamba1 max size", case, "fast kernel" if below else "token loop", "row bytes", L * Dc * 2)
    inp = gen.make_mamba1(b, L, Dc, 16, act="bf16", seed=L % 1000, gate=True, h0=True)
    a = "bf16"
    y, h, _ = bd.sscan_mamba1_fwd(dev(inp.x, a), dev(inp.dt_raw, a), par(inp.dt_bias), par(inp.A_log),
                                  dev(inp.B, a), dev(inp.C, a), par(inp.D), dev(inp.z, a), par(inp.h0))
    torch.cuda.synchronize()
    chans = [0, 1, 5, Dc // 2 - 1, Dc - 4, Dc - 1]
    got = (_pick(y, chans, 2), _pick(h, chans, 1))
    del y, h
    torch.cuda.empty_cache()
    sub = _mamba1_subset(inp, chans)
    del inp
    say("  oracle on channels", chans)
    check_all(sub, got, oracle.run_inputs(sub), "mamba1")


# batch, seqlen, heads, state_dim: one token below and one past a 2^31-byte batch row of x
SSD_MAX = [(2, ROW_LIMIT // (80 * 64 * 2) - 0, 80, 128), (1, ROW_LIMIT // (80 * 64 * 2) + 1, 80, 64)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", SSD_MAX, ids=lambda c: "b%d_L%d_H%d_N%d" % c)
def test_ssd_largest_rows(case):
    b, L, H, N = case
    below = L * H * 64 * 2 < ROW_LIMIT
    say("ssd max size", case, "chunk kernel" if below else "token loop", "row bytes", L * H * 64 * 2)
    inp = gen.make_ssd(b, L, H, 64, N, act="bf16", seed=L % 1000, gate=True, h0=True)
    a = "bf16"
    x, B = dev(inp.x, a), dev(inp.B, a)
    need = bd.sscan_ssd_workspace_size(bd.ssd_desc(x, B))
    work = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    y, h, _ = bd.sscan_ssd_fwd(x, dev(inp.dt_raw, a), par(inp.dt_bias), par(inp.A_log), B, dev(inp.C, a),
                               par(inp.D), dev(inp.z, a), par(inp.h0), workspace=work)
    torch.cuda.synchronize()
    if below:
        o = bd.SSD_GIVEUP_WORD_OFFSET
        assert int(work[o:o + 4].cpu().numpy().view(np.uint32)[0]) == 0
    heads = [0, H // 2, H - 1]
    got = (_pick(y, heads, 2), _pick(h, heads, 1))
    del x, B, y, h, work
    torch.cuda.empty_cache()
    sub = _ssd_subset(inp, heads)
    del inp
    say("  oracle on heads", heads)
    check_all(sub, got, oracle.run_inputs(sub), "ssd" if below else "mamba1")
