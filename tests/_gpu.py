"""Helpers for the GPU parity tests: upload generator inputs, run the HIP path
through the C ABI binding, and compare with the oracle under the stated rules."""
import sys

import numpy as np
import torch

from state_space_model_sscan_amd import binding as bd

# Tolerances: fp32 inputs: max|diff| <= 1e-4 * max|ref|; bf16 inputs with fp32
# accumulation, compared on the same bf16-rounded inputs: relative L2 <= 5e-3.
FP32_MAXREL = 1e-4
BF16_RELL2 = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, act, device="cuda:0"):
    """numpy float32 (bf16-representable when act == 'bf16') -> torch tensor on the GPU."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if act == "bf16":
        t = t.to(torch.bfloat16)  # exact: the values are already bf16
    return t.to(device)


def par(a, device="cuda:0"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def run_mamba1(inp, want_states=None, state_input=None):
    ws = inp.want_states if want_states is None else want_states
    a = inp.act
    y, h, st = bd.sscan_mamba1_fwd(dev(inp.x, a), dev(inp.dt_raw, a), par(inp.dt_bias), par(inp.A_log),
                                   dev(inp.B, a), dev(inp.C, a), par(inp.D), dev(inp.z, a),
                                   par(inp.h0 if state_input is None else state_input),
                                   bc_rms_eps=inp.bc_eps, want_states=ws)
    torch.cuda.synchronize()
    return host(y), host(h), host(st)


def run_ssd(inp, want_states=None, chunk=0):
    ws = inp.want_states if want_states is None else want_states
    a = inp.act
    y, h, st = bd.sscan_ssd_fwd(dev(inp.x, a), dev(inp.dt_raw, a), par(inp.dt_bias), par(inp.A_log),
                                dev(inp.B, a), dev(inp.C, a), par(inp.D), dev(inp.z, a), par(inp.h0),
                                want_states=ws, chunk=chunk)
    torch.cuda.synchronize()
    return host(y), host(h), host(st)


def max_rel(got, ref):
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err / scale if scale > 0 else err


def rel_l2(got, ref):
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((got - ref).ravel()))
    return num / den if den > 0 else num


def check(got, ref, act, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s has non-finite values" % what
    if act == "bf16":
        e = rel_l2(got, ref)
        say("  %-14s rel_l2 %.3e (limit %.0e)" % (what, e, BF16_RELL2))
        assert e <= BF16_RELL2, (what, e)
    else:
        e = max_rel(got, ref)
        say("  %-14s max|d|/max|ref| %.3e (limit %.0e)" % (what, e, FP32_MAXREL))
        assert e <= FP32_MAXREL, (what, e)
    return e


def sample_channels(Dc, k, seed=0):
    """A spread of channels: both ends of the first, a middle and the last 64-lane block, plus random ones."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, Dc // 2, Dc - 65, Dc - 64, Dc - 1]
    pick = set(c for c in fixed if 0 <= c < Dc)
    while len(pick) < min(k, Dc):
        pick.add(int(rng.integers(0, Dc)))
    return np.array(sorted(pick))


def mamba1_subset(inp, sel):
    """The same problem restricted to channels `sel` (channels are independent given B, C)."""
    import copy
    s = copy.copy(inp)
    s.x = inp.x[:, :, sel]
    s.dt_raw = inp.dt_raw[:, :, sel]
    s.z = None if inp.z is None else inp.z[:, :, sel]
    s.dt_bias = inp.dt_bias[sel]
    s.A_log = inp.A_log[sel]
    s.D = inp.D[sel]
    s.h0 = None if inp.h0 is None else inp.h0[:, sel]
    s.channels = len(sel)
    return s


def ssd_subset(inp, heads):
    import copy
    s = copy.copy(inp)
    s.x = inp.x[:, :, heads]
    s.z = None if inp.z is None else inp.z[:, :, heads]
    s.dt_raw = inp.dt_raw[:, :, heads]
    s.dt_bias = inp.dt_bias[heads]
    s.A_log = inp.A_log[heads]
    s.D = inp.D[heads]
    s.h0 = None if inp.h0 is None else inp.h0[:, heads]
    s.nheads = len(heads)
    return s
