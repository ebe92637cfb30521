"""GPU parity of the steps next to the scan, the Mamba-2 decode step, the SSD scan with
fp32 activations and the hidden attention map at the shapes the benchmark times (the
Mamba-2 2.7B layer: batch 4, 8192 tokens, 80 heads x 64, state 128, xBC width 5376), in
the same launch configuration. The conv, the norm and the decode step are compared whole. The
attention map (1.3 GB of fp32 at 2048 tokens) is compared on windows: an entry
alpha[t, s] depends only on tokens s..t, so the oracle's map of the subsequence
[s1, t2) holds alpha[t, s] for s1 <= s <= t < t2."""
import numpy as np
import pytest
import torch

import oracle
from state_space_model_sscan_amd import binding as bd
from state_space_model_sscan_amd import inputs as gen

from _gpu import check, check_all, dev, host, par, run_ssd, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


@pytest.mark.timeout(600)
def test_conv1d_at_the_2p7b_xbc_shape():
    b, L, Dc, W = 4, 8192, 5376, 4
    say("conv at", (b, L, Dc, W))
    g = torch.Generator(device="cuda")
    g.manual_seed(5376)
    x = torch.randn((b, L, Dc), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((Dc, W), generator=g, device="cuda") * 0.5).contiguous()
    bias = torch.randn((Dc,), generator=g, device="cuda") * 0.1
    st = torch.randn((b, Dc, W - 1), generator=g, device="cuda")
    out, st_out = bd.sscan_conv1d_silu(x, w, bias, st)
    torch.cuda.synchronize()
    ref, ref_st = oracle.conv1d_silu(host(x), host(w), host(bias), host(st))
    check(host(out), ref, "bf16", "conv out", path="stream")
    assert np.array_equal(host(st_out), ref_st.astype(np.float32).astype(np.float64))


@pytest.mark.timeout(600)
def test_gated_norm_at_the_2p7b_shape():
    rows, width = 4 * 8192, 5120
    say("gated norm at", (rows, width))
    g = torch.Generator(device="cuda")
    g.manual_seed(5120)
    y = torch.randn((rows, width), generator=g, device="cuda").to(torch.bfloat16)
    z = torch.randn((rows, width), generator=g, device="cuda").to(torch.bfloat16)
    wt = torch.rand((width,), generator=g, device="cuda") + 0.5
    out = bd.sscan_gated_rmsnorm(y, z, wt, 1e-5)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(host(y), host(z), host(wt), 1e-5)
    check(host(out), ref, "bf16", "norm out", path="stream")


@pytest.mark.timeout(600)
def test_ssd_fp32_at_the_2p7b_shape():
    """fp32 activations at the 2.7B layer shape, one batch row (the fp32 MFMA chunk path
    the benchmark times), every element of y and of the final state."""
    inp = gen.make_workload(4, batch=1, act="f32")
    say("ssd fp32 at", (1, inp.seqlen, inp.nheads, inp.head_dim, inp.state_dim))
    got = run_ssd(inp)
    check_all(inp, got, oracle.run_inputs(inp), "ssd")


def test_ssd_fp32_four_rows_at_the_2p7b_width():
    """fp32 activations on all four batch rows at the 2.7B width (320 chains, the plan the
    benchmark's full-batch fp32 figure runs), 2048 tokens, every element."""
    inp = gen.make_ssd(4, 2048, 80, 64, 128, act="f32", seed=2704, gate=True, h0=True)
    say("ssd fp32 four rows", (4, inp.seqlen, inp.nheads, inp.head_dim, inp.state_dim))
    check_all(inp, run_ssd(inp), oracle.run_inputs(inp), "ssd")


def test_ssd_decode_step_at_the_2p7b_shape():
    """Two one-token steps at batch 4 x 80 heads x 64 x 128, the state updated in place,
    against the oracle's scan of the same two tokens from the same state."""
    inp = gen.make_ssd(4, 2, 80, 64, 128, act="bf16", seed=2702, gate=True, h0=True)
    say("ssd decode at", inp.x.shape)
    yr, hr, _ = oracle.run_inputs(inp)
    state = par(inp.h0).clone()
    ys = []
    for t in range(2):
        one = lambda a: dev(a[:, t:t + 1], "bf16")
        y, _ = bd.sscan_ssd_step(state, one(inp.x), one(inp.dt_raw), par(inp.dt_bias), par(inp.A_log), one(inp.B),
                                 one(inp.C), par(inp.D), one(inp.z), state_output=state)
        ys.append(host(y))
    torch.cuda.synchronize()
    check_all(inp, (np.concatenate(ys, 1), host(state)), (yr, hr), "mamba1")


def test_attention_map_at_2048_tokens_sampled_windows():
    L, H = 2048, 80
    inp = gen.make_ssd(1, L, H, 64, 128, act="bf16", seed=2048, gate=False, h0=False, zero_step_frac=0.01)
    say("attention map at", (1, L, L, H))
    alpha = bd.sscan_ssd_attention(dev(inp.dt_raw, "bf16"), par(inp.dt_bias), par(inp.A_log),
                                   dev(inp.B, "bf16"), dev(inp.C, "bf16"))
    torch.cuda.synchronize()
    for s1, t2 in ((0, 96), (1000, 1070), (1950, 2048)):
        sub = oracle.ssd_attention(inp.dt_raw[:, s1:t2], inp.dt_bias, inp.A_log, inp.B[:, s1:t2], inp.C[:, s1:t2])
        got = host(alpha[:, s1:t2, s1:t2])
        check(got, sub, "f32", "alpha window [%d, %d)" % (s1, t2))
    # whole rows, far keys included: the zeros above the diagonal, and rows that
    # reach back to token 0 against the oracle's map of the first tokens
    for t in (5, 700, 2047):
        row = host(alpha[0, t])
        assert np.all(row[t + 1:] == 0.0)
    head = oracle.ssd_attention(inp.dt_raw[:, :160], inp.dt_bias, inp.A_log, inp.B[:, :160], inp.C[:, :160])
    check(host(alpha[:, :160, :160]), head, "f32", "alpha, first 160 tokens")
