"""The C ABI on the CPU: the library loads, exports every declared symbol, and
every validation path returns its status before any launch (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from state_space_model_sscan_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sscan.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sscan_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = bd.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(bd.EXPORTS)
    assert L.sscan_abi_version() == 3


def test_status_strings():
    L = bd.lib()
    assert L.sscan_status_string(0) == b"ok"
    assert L.sscan_status_string(4) == b"unsupported variant"
    assert L.sscan_status_string(99) == b"unknown status"


class Host:
    """16-byte aligned host buffers whose addresses stand in for tensors."""

    def __init__(self):
        self.keep = []

    def buf(self, nbytes):
        a = np.zeros(max(int(nbytes), 1) + 64, np.uint8)
        off = (-a.ctypes.data) % 64
        self.keep.append(a)
        return a.ctypes.data + off


def m1_args(h, d, ws=0):
    es = 2 if d.act == 1 else 4
    b, L, Dc, N, G = d.batch, d.seqlen, d.channels, d.state_dim, d.ngroups
    act = b * L * Dc * es
    return dict(x=h.buf(act), dt=h.buf(act), bias=h.buf(Dc * 4), alog=h.buf(Dc * N * 4), B=h.buf(b * L * G * N * es),
                C=h.buf(b * L * G * N * es), D=h.buf(Dc * 4), z=h.buf(act), h0=h.buf(b * Dc * N * 4), y=h.buf(act),
                hout=h.buf(b * Dc * N * 4), states=None, ws=h.buf(ws) if ws else None, wsb=ws)


def call_m1(d, a):
    L = bd.lib()
    return L.sscan_mamba1_fwd(ctypes.byref(d), a["x"], a["dt"], a["bias"], a["alog"], a["B"], a["C"], a["D"],
                              a["z"], a["h0"], a["y"], a["hout"], a["states"], a["ws"], a["wsb"], None)


def desc(**kw):
    base = dict(batch=2, seqlen=8, channels=128, state_dim=16, ngroups=1, act=0, bc_rms_eps=0.0)
    base.update(kw)
    return bd.Mamba1Desc(**base)


def status(code):
    return bd.STATUS_NAMES[code]


def test_null_descriptor():
    L = bd.lib()
    assert status(L.sscan_mamba1_fwd(None, *([None] * 13), 0, None)) == "SSCAN_ERR_NULL"
    assert status(L.sscan_ssd_fwd(None, *([None] * 13), 0, None)) == "SSCAN_ERR_NULL"
    assert L.sscan_mamba1_workspace_size(None) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(batch=-1), "SSCAN_ERR_SHAPE"),
    (dict(channels=0), "SSCAN_ERR_SHAPE"),
    (dict(state_dim=0), "SSCAN_ERR_SHAPE"),
    (dict(ngroups=3), "SSCAN_ERR_SHAPE"),
    (dict(act=7), "SSCAN_ERR_DTYPE"),
    (dict(state_dim=257), "SSCAN_ERR_UNSUPPORTED"),
    (dict(channels=192, ngroups=2), "SSCAN_ERR_UNSUPPORTED"),
    (dict(batch=70000), "SSCAN_ERR_UNSUPPORTED"),
])
def test_mamba1_descriptor_errors(kw, want):
    h = Host()
    d = desc(**kw)
    if d.batch >= 0 and d.channels > 0 and 0 < d.state_dim <= 256 and d.batch < 70000:
        a = m1_args(h, d)
    else:
        a = m1_args(h, desc())
    assert status(call_m1(d, a)) == want
    assert bd.lib().sscan_last_error()


def test_mamba1_pointer_errors():
    h = Host()
    d = desc()
    a = m1_args(h, d)
    a["x"] = None
    assert status(call_m1(d, a)) == "SSCAN_ERR_NULL"
    a = m1_args(h, d)
    a["B"] += 4
    assert status(call_m1(d, a)) == "SSCAN_ERR_ALIGN"
    a = m1_args(h, d)
    a["y"] = a["x"]
    assert status(call_m1(d, a)) == "SSCAN_ERR_ALIAS"
    a = m1_args(h, d)
    a["hout"] = a["h0"]                        # in place is for the decode step only
    assert status(call_m1(d, a)) == "SSCAN_ERR_ALIAS"
    a = m1_args(h, d)                          # host memory is refused
    assert status(call_m1(d, a)) == "SSCAN_ERR_NOT_DEVICE"
    # optional inputs may be NULL
    a = m1_args(h, d)
    a["z"] = a["h0"] = None
    assert status(call_m1(d, a)) == "SSCAN_ERR_NOT_DEVICE"


def test_mamba1_workspace():
    h = Host()
    # one batch row of 128 channels over a long sequence is cut into slices
    d = desc(batch=1, seqlen=16384, channels=128)
    need = bd.lib().sscan_mamba1_workspace_size(ctypes.byref(d))
    assert need > 0 and need % 4 == 0
    # the query is a pure function of the shape
    assert need == bd.lib().sscan_mamba1_workspace_size(ctypes.byref(desc(batch=1, seqlen=16384, channels=128)))
    # the Mamba-130m layer shape fills the chip without slices
    assert bd.lib().sscan_mamba1_workspace_size(ctypes.byref(desc(batch=8, seqlen=2048, channels=1536))) == 0
    a = m1_args(h, d, ws=need - 4)
    assert status(call_m1(d, a)) == "SSCAN_ERR_WORKSPACE"
    a = m1_args(h, d, ws=0)
    assert status(call_m1(d, a)) == "SSCAN_ERR_WORKSPACE"
    a = m1_args(h, d, ws=need)
    assert status(call_m1(d, a)) == "SSCAN_ERR_NOT_DEVICE"
    # short sequences need none
    assert bd.lib().sscan_mamba1_workspace_size(ctypes.byref(desc(seqlen=64))) == 0


def test_step_errors_and_in_place():
    L = bd.lib()
    h = Host()
    d = desc(seqlen=2)
    a = m1_args(h, desc(seqlen=1))
    args = lambda a: (a["h0"], a["hout"], a["x"], a["dt"], a["bias"], a["alog"], a["B"], a["C"], a["D"], a["z"],
                      a["y"], None)
    assert status(L.sscan_step(ctypes.byref(d), *args(a))) == "SSCAN_ERR_SHAPE"
    d = desc(seqlen=1)
    a["hout"] = a["h0"]                        # in place is allowed for a step
    assert status(L.sscan_step(ctypes.byref(d), *args(a))) == "SSCAN_ERR_NOT_DEVICE"
    a2 = dict(a)
    a2["hout"] = a["h0"] + 16                  # a partial overlap is not
    assert status(L.sscan_step(ctypes.byref(d), *args(a2))) == "SSCAN_ERR_ALIAS"
    a3 = dict(a)
    a3["h0"] = None                            # a step needs its entering state
    a3["hout"] = h.buf(2 * 128 * 16 * 4)
    assert status(L.sscan_step(ctypes.byref(d), *args(a3))) == "SSCAN_ERR_NULL"


def sdesc(**kw):
    base = dict(batch=2, seqlen=32, nheads=4, head_dim=64, state_dim=128, ngroups=1, chunk=0, act=1, reserved=0)
    base.update(kw)
    return bd.SSDDesc(**base)


@pytest.mark.parametrize("kw,want", [
    (dict(nheads=0), "SSCAN_ERR_SHAPE"),
    (dict(ngroups=3), "SSCAN_ERR_SHAPE"),
    (dict(chunk=100), "SSCAN_ERR_SHAPE"),
    (dict(chunk=512), "SSCAN_ERR_SHAPE"),
    (dict(reserved=1), "SSCAN_ERR_SHAPE"),
    (dict(act=2), "SSCAN_ERR_DTYPE"),
    (dict(state_dim=256), "SSCAN_ERR_UNSUPPORTED"),
    (dict(nheads=4, head_dim=8, ngroups=2), "SSCAN_ERR_UNSUPPORTED"),
])
def test_ssd_descriptor_errors(kw, want):
    L = bd.lib()
    h = Host()
    d = sdesc(**kw)
    ptrs = [h.buf(1 << 20) for _ in range(13)]
    ptrs[11] = None
    assert status(L.sscan_ssd_fwd(ctypes.byref(d), *ptrs, 1 << 20, None)) == want


def test_ssd_host_pointers_refused():
    L = bd.lib()
    h = Host()
    d = sdesc()
    b, Ln, H, P, N = 2, 32, 4, 64, 128
    act = b * Ln * H * P * 2
    ws = L.sscan_ssd_workspace_size(ctypes.byref(d))
    ptrs = [h.buf(act), h.buf(b * Ln * H * 2), h.buf(H * 4), h.buf(H * 4), h.buf(b * Ln * N * 2),
            h.buf(b * Ln * N * 2), h.buf(H * 4), None, None, h.buf(act), h.buf(b * H * P * N * 4), None,
            h.buf(ws) if ws else None]
    assert status(L.sscan_ssd_fwd(ctypes.byref(d), *ptrs, ws, None)) == "SSCAN_ERR_NOT_DEVICE"
    # the pointer check can be switched off; the previous setting is returned
    assert bd.set_pointer_checks(True) is True


def test_conv_and_norm_errors():
    L = bd.lib()
    h = Host()
    d = bd.ConvDesc(2, 8, 64, 4, 0, 0)
    p = [h.buf(2 * 8 * 64 * 4), h.buf(64 * 4 * 4), None, None, h.buf(2 * 8 * 64 * 4), None]
    assert status(L.sscan_conv1d_silu(ctypes.byref(d), *p, None)) == "SSCAN_ERR_NOT_DEVICE"
    assert status(L.sscan_conv1d_silu(ctypes.byref(bd.ConvDesc(2, 8, 64, 9, 0, 0)), *p, None)) == "SSCAN_ERR_UNSUPPORTED"
    assert status(L.sscan_conv1d_silu(ctypes.byref(bd.ConvDesc(2, 8, 64, 0, 0, 0)), *p, None)) == "SSCAN_ERR_SHAPE"
    assert status(L.sscan_conv1d_silu(ctypes.byref(bd.ConvDesc(2, 8, 64, 4, 3, 0)), *p, None)) == "SSCAN_ERR_DTYPE"
    assert status(L.sscan_conv1d_silu(None, *p, None)) == "SSCAN_ERR_NULL"
    q = list(p)
    q[4] = q[0]
    assert status(L.sscan_conv1d_silu(ctypes.byref(d), *q, None)) == "SSCAN_ERR_ALIAS"
    y, z, w, o = h.buf(4 * 64 * 4), h.buf(4 * 64 * 4), h.buf(64 * 4), h.buf(4 * 64 * 4)
    assert status(L.sscan_gated_rmsnorm(4, 64, 0, y, z, w, 1e-5, o, None)) == "SSCAN_ERR_NOT_DEVICE"
    assert status(L.sscan_gated_rmsnorm(4, 64, 0, y, z, w, 0.0, o, None)) == "SSCAN_ERR_SHAPE"
    assert status(L.sscan_gated_rmsnorm(4, 0, 0, y, z, w, 1e-5, o, None)) == "SSCAN_ERR_SHAPE"
    assert status(L.sscan_gated_rmsnorm(4, 64, 5, y, z, w, 1e-5, o, None)) == "SSCAN_ERR_DTYPE"
    assert status(L.sscan_gated_rmsnorm(4, 64, 0, y, z, w, 1e-5, y, None)) == "SSCAN_ERR_ALIAS"


def test_attention_workspace_and_pointers():
    """sscan_ssd_attention: the workspace query, a missing or short workspace, host
    pointers, and a workspace that overlaps the map, all refused before any launch."""
    L = bd.lib()
    h = Host()
    b, Ln, H, N, G = 2, 40, 8, 16, 2
    d = bd.SSDDesc(b, Ln, H, 1, N, G, 0, 0, 0)
    need = L.sscan_ssd_attention_workspace_size(ctypes.byref(d))
    assert need == b * Ln * H * 12
    p = [h.buf(b * Ln * H * 4), h.buf(H * 4), h.buf(H * 4), h.buf(b * Ln * G * N * 4), h.buf(b * Ln * G * N * 4),
         h.buf(b * Ln * Ln * H * 4)]
    ws = h.buf(need)
    assert status(L.sscan_ssd_attention(ctypes.byref(d), *p, None, 0, None)) == "SSCAN_ERR_WORKSPACE"
    assert status(L.sscan_ssd_attention(ctypes.byref(d), *p, ws, need - 1, None)) == "SSCAN_ERR_WORKSPACE"
    assert status(L.sscan_ssd_attention(ctypes.byref(d), *p, ws, need, None)) == "SSCAN_ERR_NOT_DEVICE"
    assert status(L.sscan_ssd_attention(ctypes.byref(d), *p, p[5], need, None)) == "SSCAN_ERR_ALIAS"
    bad = bd.SSDDesc(b, Ln, H, 1, N, 3, 0, 0, 0)   # 3 groups do not divide 8 heads
    assert L.sscan_ssd_attention_workspace_size(ctypes.byref(bad)) == 0
    assert status(L.sscan_ssd_attention(ctypes.byref(bad), *p, ws, need, None)) == "SSCAN_ERR_SHAPE"


def test_tuning_knobs_are_validated_and_restored():
    L = bd.lib()
    assert L.sscan_set_tuning(99, 1) == -1          # unknown knob: nothing changes
    assert L.sscan_set_tuning(0, 1) == -1
    assert L.sscan_set_tuning(bd.TUNE_M1_LANES, -2) == -1
    assert bd.set_tuning(bd.TUNE_M1_LANES, 4) == 0
    assert bd.set_tuning(bd.TUNE_M1_LANES, 0) == 4   # the previous value comes back
    assert bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, 1) == 0
    assert bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, 0) == 1
    assert bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 2) == 0
    assert bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 0) == 2
    assert bd.set_tuning(bd.TUNE_SSD_SPLIT_STATE, 1) == 0
    assert bd.set_tuning(bd.TUNE_SSD_SPLIT_STATE, 0) == 1
    assert L.sscan_set_tuning(bd.TUNE_SSD_SPLIT_STATE + 1, 1) == -1   # one past the last knob
    with pytest.raises(ValueError):
        bd.set_tuning(42, 1)


def test_launch_plans_are_stable_and_follow_the_knobs():
    """The workspace queries are pure functions of the shape and the knobs: repeated
    queries agree, a knob changes the plan only while it is set, and a call whose
    workspace was sized under another setting is refused, not run."""
    L = bd.lib()
    m = desc(batch=1, seqlen=16384, channels=128)
    # many heads, few chunks: the chunk path's workspace is the larger of the two SSD paths'
    s = sdesc(batch=1, seqlen=256, nheads=400)
    m0 = L.sscan_mamba1_workspace_size(ctypes.byref(m))
    s0 = L.sscan_ssd_workspace_size(ctypes.byref(s))
    for _ in range(3):
        assert L.sscan_mamba1_workspace_size(ctypes.byref(m)) == m0
        assert L.sscan_ssd_workspace_size(ctypes.byref(s)) == s0
    # one segment per chain: no state hand-off buffer
    bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 64)
    try:
        one = L.sscan_ssd_workspace_size(ctypes.byref(s))
        bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 1)
        many = L.sscan_ssd_workspace_size(ctypes.byref(s))
        assert many == one + 400 * 64 * 128 * 4       # the hand-off states of 400 chains
        # a workspace sized for one segment per chain is too small for one-chunk segments
        h = Host()
        b, Ln, H, P, N = 1, 256, 400, 64, 128
        act = b * Ln * H * P * 2
        ptrs = [h.buf(act), h.buf(b * Ln * H * 2), h.buf(H * 4), h.buf(H * 4), h.buf(b * Ln * N * 2),
                h.buf(b * Ln * N * 2), h.buf(H * 4), None, None, h.buf(act), h.buf(b * H * P * N * 4), None,
                h.buf(one)]
        assert status(L.sscan_ssd_fwd(ctypes.byref(s), *ptrs, one, None)) == "SSCAN_ERR_WORKSPACE"
    finally:
        bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 0)
    assert L.sscan_ssd_workspace_size(ctypes.byref(s)) == s0
    # fp32 activations take the fp32 chunk kernel (its plan: the larger workspace here)
    # unless the knob sends them to the token loop
    f = sdesc(batch=1, seqlen=256, nheads=400, act=0)
    f0 = L.sscan_ssd_workspace_size(ctypes.byref(f))
    bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, 1)
    try:
        ft = L.sscan_ssd_workspace_size(ctypes.byref(f))
    finally:
        bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, 0)
    assert ft < f0   # (400 heads need no slices on the token loop: no workspace at all)
    # a sequence of length 0 takes no chunk-path workspace: the call only passes the state through
    assert L.sscan_ssd_workspace_size(ctypes.byref(sdesc(seqlen=0))) == 0
    assert L.sscan_ssd_workspace_size(ctypes.byref(sdesc(seqlen=0, act=0))) == 0
    assert L.sscan_ssd_workspace_size(ctypes.byref(f)) == f0
    # 16 heads of one batch row (16 chains for 256 units) take two passes: the first
    # pass's states and decay sums make the workspace larger than one pass's
    few = sdesc(batch=1, seqlen=16384, nheads=16)
    w_plan = L.sscan_ssd_workspace_size(ctypes.byref(few))
    for v, want in ((2, w_plan), (0, w_plan)):
        bd.set_tuning(bd.TUNE_SSD_TWO_PASS, v)
        assert L.sscan_ssd_workspace_size(ctypes.byref(few)) == want
    bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 1)
    try:
        assert L.sscan_ssd_workspace_size(ctypes.byref(few)) < w_plan
    finally:
        bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 0)
    # four batch rows (320 chains) keep one pass
    many = sdesc(batch=4, seqlen=8192, nheads=80)
    w4 = L.sscan_ssd_workspace_size(ctypes.byref(many))
    bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 1)
    try:
        assert L.sscan_ssd_workspace_size(ctypes.byref(many)) == w4
    finally:
        bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 0)
    # a head of 128 or 256 columns is planned as 2 or 4 heads of 64 columns
    for act in (1, 0):
        for P, m in ((128, 2), (256, 4)):
            wide = sdesc(batch=2, seqlen=3000, nheads=40, head_dim=P, act=act)
            narrow = sdesc(batch=2, seqlen=3000, nheads=40 * m, head_dim=64, act=act)
            assert L.sscan_ssd_workspace_size(ctypes.byref(wide)) == L.sscan_ssd_workspace_size(ctypes.byref(narrow))


def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.float32)


def test_binding_refuses_misshaped_tensors():
    """The C ABI cannot see buffer sizes, so the binding checks every tensor's shape
    and raises before anything reaches the library."""
    import torch
    b, L, Dc, N = 2, 8, 64, 16
    ok = dict(x=_cpu(b, L, Dc), dt_raw=_cpu(b, L, Dc), dt_bias=_cpu(Dc), A_log=_cpu(Dc, N), B=_cpu(b, L, 1, N),
              C=_cpu(b, L, 1, N), D=_cpu(Dc))
    bad = [("dt_raw", _cpu(b, L, Dc + 1)), ("dt_bias", _cpu(Dc - 1)), ("A_log", _cpu(N, Dc)), ("C", _cpu(b, L, 1, 8)),
           ("D", _cpu(1)), ("z", _cpu(b, L - 1, Dc)), ("state_input", _cpu(b, Dc, N + 1)), ("y", _cpu(b, L, Dc, 1)),
           ("state_output", _cpu(b, N, Dc)), ("states", _cpu(b, L, Dc, 8))]
    for name, t in bad:
        kw = dict(ok)
        kw[name] = t
        with pytest.raises(ValueError, match=name):
            bd.sscan_mamba1_fwd(**kw)
    with pytest.raises(TypeError):
        bd.sscan_mamba1_fwd(**ok, y=_cpu(b, L, Dc, dtype=torch.bfloat16))
    # the decode step
    one = dict(x=_cpu(b, 1, Dc), dt_raw=_cpu(b, 1, Dc), dt_bias=_cpu(Dc), A_log=_cpu(Dc, N), B=_cpu(b, 1, 1, N),
               C=_cpu(b, 1, 1, N), D=_cpu(Dc))
    with pytest.raises(ValueError, match="state_input"):
        bd.sscan_step(_cpu(b, Dc, N - 1), **one)
    with pytest.raises(ValueError, match="one token"):
        bd.sscan_step(_cpu(b, Dc, N), **dict(one, x=_cpu(b, 2, Dc)))
    # SSD
    H, P, Ns = 4, 64, 128
    s_ok = dict(x=_cpu(b, L, H, P), dt_raw=_cpu(b, L, H), dt_bias=_cpu(H), A_log=_cpu(H), B=_cpu(b, L, 1, Ns),
                C=_cpu(b, L, 1, Ns), D=_cpu(H))
    for name, t in [("dt_raw", _cpu(b, L, H, 1)), ("A_log", _cpu(H, 1)), ("z", _cpu(b, L, H, P + 1)),
                    ("state_input", _cpu(b, H, Ns, P)), ("state_output", _cpu(b, H, Ns, P)),
                    ("states", _cpu(b, L, H, P, 1))]:
        with pytest.raises(ValueError, match=name):
            bd.sscan_ssd_fwd(**dict(s_ok, **{name: t}))
    with pytest.raises(ValueError, match="state_input"):
        bd.sscan_ssd_step(_cpu(b, H, P, Ns + 1), **{k: (v[:, :1].contiguous() if k in ("x", "dt_raw", "B", "C") else v)
                                                    for k, v in s_ok.items()})
    # attention map, conv, norm
    with pytest.raises(ValueError, match="alpha"):
        bd.sscan_ssd_attention(_cpu(b, L, H), _cpu(H), _cpu(H), _cpu(b, L, 1, 16), _cpu(b, L, 1, 16), alpha=_cpu(b, L, L))
    with pytest.raises(ValueError, match="weight"):
        bd.sscan_conv1d_silu(_cpu(b, L, Dc), _cpu(Dc + 1, 4))
    with pytest.raises(ValueError, match="conv_state_in"):
        bd.sscan_conv1d_silu(_cpu(b, L, Dc), _cpu(Dc, 4), conv_state_in=_cpu(b, Dc, 4))
    with pytest.raises(ValueError, match="z"):
        bd.sscan_gated_rmsnorm(_cpu(4, 64), _cpu(4, 65), _cpu(64), 1e-5)
    with pytest.raises(ValueError, match="weight"):
        bd.sscan_gated_rmsnorm(_cpu(4, 64), _cpu(4, 64), _cpu(63), 1e-5)


# A C consumer of the header: prints the descriptor layouts, the constants and what
# the library answers without a GPU (version, status text, a workspace query).
_C_CONSUMER = r"""
#include <stddef.h>
#include <stdio.h>
#include "sscan.h"
#define OFF(T, f) (long)offsetof(T, f)
int main(void) {
  sscan_mamba1_desc m = {8, 2048, 1536, 16, 1, SSCAN_BF16, 0.0f};
  printf("mamba1 %ld %ld %ld %ld\n", (long)sizeof(sscan_mamba1_desc), OFF(sscan_mamba1_desc, ngroups),
         OFF(sscan_mamba1_desc, act), OFF(sscan_mamba1_desc, bc_rms_eps));
  printf("ssd %ld %ld %ld %ld\n", (long)sizeof(sscan_ssd_desc), OFF(sscan_ssd_desc, chunk),
         OFF(sscan_ssd_desc, act), OFF(sscan_ssd_desc, reserved));
  printf("conv %ld %ld %ld %ld\n", (long)sizeof(sscan_conv_desc), OFF(sscan_conv_desc, width),
         OFF(sscan_conv_desc, act), OFF(sscan_conv_desc, reserved));
  printf("consts %d %d %u\n", SSCAN_ABI_VERSION, SSCAN_SSD_GIVEUP_WORD_OFFSET, (unsigned)SSCAN_NOALLOC_SCRATCH_BYTES);
  printf("version %d\n", sscan_abi_version());
  printf("status %s\n", sscan_status_string(SSCAN_ERR_ALIGN));
  printf("workspace %zu\n", sscan_mamba1_workspace_size(&m));
  return 0;
}
"""


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_is_plain_c_and_matches_the_binding(tmp_path, lang):
    """include/sscan.h compiles on its own as strict C99 and as C++ (extern "C"), a
    program built against it links to libsscan.so and runs without a GPU, and the
    descriptor layouts it sees are the ones the ctypes binding passes."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    src = tmp_path / ("consumer.c" if lang == "c" else "consumer.cpp")
    src.write_text(_C_CONSUMER)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(bd.LIB_PATH)
    std = ["-std=c99", "-pedantic"] if lang == "c" else ["-std=c++17"]
    cmd = [cc, *std, "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           bd.LIB_PATH, "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    for name, cls, fields in (("mamba1", bd.Mamba1Desc, ("ngroups", "act", "bc_rms_eps")),
                              ("ssd", bd.SSDDesc, ("chunk", "act", "reserved")),
                              ("conv", bd.ConvDesc, ("width", "act", "reserved"))):
        want = [ctypes.sizeof(cls)] + [getattr(cls, f).offset for f in fields]
        assert [int(v) for v in out[name].split()] == want, (name, out[name], want)
    assert out["consts"].split() == ["3", str(bd.SSD_GIVEUP_WORD_OFFSET), str(16 << 20)]
    assert out["version"] == "3"
    assert out["status"] == bd.lib().sscan_status_string(6).decode()
    d = bd.Mamba1Desc(8, 2048, 1536, 16, 1, bd.BF16, 0.0)
    assert int(out["workspace"]) == bd.sscan_mamba1_workspace_size(d)
