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
# bf16 results are also checked element by element, so that a few wrong values
# cannot hide in the relative L2 of millions:
#     |got_i - ref_i| <= 2^-8 |ref_i| + (1 + 2^-8) k mag_i,
# where mag_i is the same scan run by the oracle on the absolute values of x, B,
# C, D and the entering state (no gate), times |silu(z_i)|: the sum of the sizes
# of every term that makes up y_i (or the state entry). bf16 keeps 8 significant
# bits, so rounding a value v to bf16 moves it by at most 2^-8 |v|; with v the
# kernel's fp32 result, |RNE(v) - ref| <= 2^-8 |ref| + (1 + 2^-8) |v - ref|, and
# |v - ref| <= k mag_i, where k is 2^-8 per bf16 rounding of an operand on a
# term's path plus the fp32 arithmetic (exp2, sums), which stays below 2^-12 of
# mag at these lengths:
#   Mamba-1 kernels and the token loop: fp32 arithmetic only, k = 2^-10;
#   SSD MFMA chunk path: two roundings on every term's path (the masked C.B^T
#   entry inside a chunk; w*x and the state as C reads it across chunks),
#   k = 2 * 2^-8.
ELEM_K = {"mamba1": 2.0 ** -10, "ssd": 2 * 2.0 ** -8}


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


def ssd_chunk_path(inp, want_states, token_loop=False):
    """Whether sscan_ssd_fwd takes the MFMA chunk path for these inputs (bf16 MFMA for
    bf16 activations, fp32 MFMA for fp32 ones; token_loop: fp32 sent to the token loop):
    head_dim 64 times a power of two, state_dim 64..128 (below 128 zero-padded), no
    per-token states."""
    m = inp.head_dim // 64
    return (inp.head_dim % 64 == 0 and m & (m - 1) == 0 and 64 <= inp.state_dim <= 128 and not want_states
            and inp.seqlen > 0 and (inp.act == "bf16" or not token_loop))


def giveup_word(workspace):
    """The chunk path's give-up word in a workspace (after a synchronize)."""
    o = bd.SSD_GIVEUP_WORD_OFFSET
    return int(workspace[o:o + 4].cpu().numpy().view(np.uint32)[0])


def run_ssd(inp, want_states=None, chunk=0, expect_giveup=False, token_loop=False):
    """sscan_ssd_fwd on the inputs; on the chunk path, the give-up word must read 0
    (or, with expect_giveup, must be raised). token_loop: fp32 activations take the
    token loop (the knob is set for the call and cleared after it)."""
    ws = inp.want_states if want_states is None else want_states
    a = inp.act
    x, B = dev(inp.x, a), dev(inp.B, a)
    prev = bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, 1 if token_loop else 0)
    try:
        need = bd.sscan_ssd_workspace_size(bd.ssd_desc(x, B, chunk))
        work = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
        y, h, st = bd.sscan_ssd_fwd(x, dev(inp.dt_raw, a), par(inp.dt_bias), par(inp.A_log), B, dev(inp.C, a),
                                    par(inp.D), dev(inp.z, a), par(inp.h0), want_states=ws, chunk=chunk,
                                    workspace=work)
        torch.cuda.synchronize()
    finally:
        bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, prev)
    if ssd_chunk_path(inp, ws, token_loop) and inp.batch > 0:
        word = giveup_word(work)
        assert (word != 0) == expect_giveup, "give-up word %d" % word
    return host(y), host(h), host(st)


def max_rel(got, ref):
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err / scale if scale > 0 else err


def rel_l2(got, ref):
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((got - ref).ravel()))
    return num / den if den > 0 else num


def magnitude(inp, want_states=False):
    """mag of the element-wise bf16 bound: the oracle's scan of the absolute values of
    x, B, C, D and the entering state, with no gate, times |silu(z)| on y.
    Returns (mag_y, mag_state, mag_states or None)."""
    import copy

    import oracle
    a = copy.copy(inp)
    a.x, a.B, a.C, a.D = np.abs(inp.x), np.abs(inp.B), np.abs(inp.C), np.abs(inp.D)
    a.h0 = None if inp.h0 is None else np.abs(inp.h0)
    a.z = None
    my, mh, ms = oracle.run_inputs(a, want_states=want_states)
    if inp.z is not None:
        z = inp.z.astype(np.float64)
        my = my * np.abs(z / (1.0 + np.exp(-z)))
    return my, mh, ms


def check(got, ref, act, what, mag=None, path="mamba1"):
    """fp32: max|d| <= 1e-4 max|ref|. bf16: relative L2 <= 5e-3 and, with mag, the
    element-wise bound |d_i| <= 2^-8 |ref_i| + k mag_i (k per path, ELEM_K)."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s has non-finite values" % what
    if act == "bf16":
        e = rel_l2(got, ref)
        d = np.abs(got - ref)
        say("  %-14s rel_l2 %.3e (limit %.0e)  max|d|/max|ref| %.3e" % (what, e, BF16_RELL2, max_rel(got, ref)))
        assert e <= BF16_RELL2, (what, e)
        if path == "stream":
            # conv1d + silu and the gated norm: a few fp32 terms per output, rounded
            # once to bf16 (at most 2^-8 of the value); the fp32 error of the terms
            # stays below 2^-16 of the largest output
            lim = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * float(np.max(np.abs(ref)))
            worst = float(np.max(d / np.maximum(lim, 1e-300)))
            say("  %-14s element-wise: worst |d|/bound %.3f" % (what, worst))
            assert np.all(d <= lim), (what, "element-wise bound", worst)
        elif mag is not None:
            k = ELEM_K[path]
            assert mag.shape == ref.shape
            lim = 2.0 ** -8 * np.abs(ref) + (1 + 2.0 ** -8) * k * mag
            worst = float(np.max(d / np.maximum(lim, 1e-300)))
            say("  %-14s element-wise: worst |d|/bound %.3f (k = %.2e)" % (what, worst, k))
            assert np.all(d <= lim), (what, "element-wise bound", worst, int(np.argmax(d - lim)))
    else:
        e = max_rel(got, ref)
        say("  %-14s max|d|/max|ref| %.3e (limit %.0e)" % (what, e, FP32_MAXREL))
        assert e <= FP32_MAXREL, (what, e)
    return e


def check_all(inp, got, ref, path, mag=None, states=False):
    """y, state_output (and per-token states) against the oracle; bf16 with the element-wise bound."""
    act = inp.act
    if act == "bf16" and mag is None:
        mag = magnitude(inp, want_states=states)
    my, mh, ms = mag if mag is not None else (None, None, None)
    check(got[0], ref[0], act, "y", my, path)
    check(got[1], ref[1], act, "state_output", mh, path)
    if states:
        check(got[2], ref[2], act, "states", ms, path)
        assert np.array_equal(got[2][:, -1], got[1]), "states[:, -1] must equal state_output bit for bit"
