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
    assert L.sscan_abi_version() == 2


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
    (dict(state_dim=129), "SSCAN_ERR_UNSUPPORTED"),
    (dict(channels=192, ngroups=2), "SSCAN_ERR_UNSUPPORTED"),
    (dict(batch=70000), "SSCAN_ERR_UNSUPPORTED"),
])
def test_mamba1_descriptor_errors(kw, want):
    h = Host()
    d = desc(**kw)
    if d.batch >= 0 and d.channels > 0 and d.state_dim > 0 and d.batch < 70000:
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
