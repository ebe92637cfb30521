"""fp64 CPU oracle for the selective scan (ctypes wrapper around sscan_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py. The product path never imports it.

All functions take numpy arrays (any float dtype; they are converted to fp64,
which is exact for fp32 and bf16 values) and return fp64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sscan_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host compiler (no HIP headers, no GPU code)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        I64, D, P = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.oracle_mamba1.argtypes = [I64] * 5 + [P] * 8 + [D] + [P] * 4
        lib.oracle_mamba1.restype = ctypes.c_int
        lib.oracle_ssd.argtypes = [I64] * 6 + [P] * 12
        lib.oracle_ssd.restype = ctypes.c_int
        lib.oracle_ssd_attention.argtypes = [I64] * 5 + [P] * 6
        lib.oracle_ssd_attention.restype = ctypes.c_int
        lib.oracle_conv1d_silu.argtypes = [I64] * 4 + [P] * 6
        lib.oracle_conv1d_silu.restype = ctypes.c_int
        lib.oracle_gated_rmsnorm.argtypes = [I64, I64, P, P, P, D, P]
        lib.oracle_gated_rmsnorm.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's later loops (the results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def mamba1(x, dt_raw, dt_bias, A_log, B, C, D, z=None, bc_eps=0.0, h0=None, want_states=False):
    """Mamba-1 scan. x: [b, L, Dc]; B, C: [b, L, G, N]; returns (y, h_out, states|None)."""
    lib = _load()
    x, dt_raw, dt_bias, A_log, B, C, D, z, h0 = map(_f64, (x, dt_raw, dt_bias, A_log, B, C, D, z, h0))
    b, L, Dc = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.empty((b, L, Dc))
    h_out = np.empty((b, Dc, N))
    states = np.empty((b, L, Dc, N)) if want_states else None
    rc = lib.oracle_mamba1(b, L, Dc, N, G, _ptr(x), _ptr(dt_raw), _ptr(dt_bias), _ptr(A_log), _ptr(B),
                           _ptr(C), _ptr(D), _ptr(z), float(bc_eps), _ptr(h0), _ptr(y), _ptr(h_out),
                           _ptr(states))
    if rc != 0:
        raise ValueError("oracle_mamba1 rejected the shapes (rc=%d)" % rc)
    return y, h_out, states


def ssd(x, dt_raw, dt_bias, A_log, B, C, D, z=None, h0=None, want_states=False):
    """Mamba-2 SSD scan. x: [b, L, H, P]; dt_raw: [b, L, H]; B, C: [b, L, G, N].
    Returns (y [b, L, H, P], h_out [b, H, P, N], states [b, L, H, P, N] | None)."""
    lib = _load()
    x, dt_raw, dt_bias, A_log, B, C, D, z, h0 = map(_f64, (x, dt_raw, dt_bias, A_log, B, C, D, z, h0))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.empty((b, L, H, P))
    h_out = np.empty((b, H, P, N))
    states = np.empty((b, L, H, P, N)) if want_states else None
    rc = lib.oracle_ssd(b, L, H, P, N, G, _ptr(x), _ptr(dt_raw), _ptr(dt_bias), _ptr(A_log), _ptr(B),
                        _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_out), _ptr(states))
    if rc != 0:
        raise ValueError("oracle_ssd rejected the shapes (rc=%d)" % rc)
    return y, h_out, states


def ssd_attention(dt_raw, dt_bias, A_log, B, C):
    """The SSD scan's hidden attention map. dt_raw: [b, L, H]; B, C: [b, L, G, N].
    Returns alpha [b, L (query), L (key), H]: y_t = sum_s alpha[t, s] x_s + D x_t before the gate."""
    lib = _load()
    dt_raw, dt_bias, A_log, B, C = map(_f64, (dt_raw, dt_bias, A_log, B, C))
    b, L, H = dt_raw.shape
    G, N = B.shape[2], B.shape[3]
    alpha = np.empty((b, L, L, H))
    rc = lib.oracle_ssd_attention(b, L, H, N, G, _ptr(dt_raw), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                  _ptr(alpha))
    if rc != 0:
        raise ValueError("oracle_ssd_attention rejected the shapes (rc=%d)" % rc)
    return alpha


def conv1d_silu(x, weight, bias=None, conv_state=None):
    """Causal depthwise conv1d + silu. x: [b, L, Dc]; weight: [Dc, W]; conv_state: [b, Dc, W-1].
    Returns (out [b, L, Dc], state_out [b, Dc, W-1])."""
    lib = _load()
    x, weight, bias, conv_state = map(_f64, (x, weight, bias, conv_state))
    b, L, Dc = x.shape
    W = weight.shape[1]
    out = np.empty((b, L, Dc))
    st = np.empty((b, Dc, max(W - 1, 0)))
    rc = lib.oracle_conv1d_silu(b, L, Dc, W, _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state),
                                _ptr(out), _ptr(st))
    if rc != 0:
        raise ValueError("oracle_conv1d_silu rejected the shapes (rc=%d)" % rc)
    return out, st


def gated_rmsnorm(y, z, weight, eps):
    """out = norm(y * silu(z)) * weight over the last axis. y, z: [..., width]."""
    lib = _load()
    y, z, weight = map(_f64, (y, z, weight))
    width = y.shape[-1]
    rows = int(np.prod(y.shape[:-1])) if y.ndim > 1 else 1
    out = np.empty(y.shape)
    rc = lib.oracle_gated_rmsnorm(rows, width, _ptr(y), _ptr(z), _ptr(weight), float(eps), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_gated_rmsnorm rejected the shapes (rc=%d)" % rc)
    return out


def run_inputs(inp, want_states=None):
    """Run the oracle on a Mamba1Inputs / SSDInputs object from the input generator."""
    ws = inp.want_states if want_states is None else want_states
    if hasattr(inp, "channels"):
        return mamba1(inp.x, inp.dt_raw, inp.dt_bias, inp.A_log, inp.B, inp.C, inp.D, inp.z,
                      inp.bc_eps, inp.h0, ws)
    return ssd(inp.x, inp.dt_raw, inp.dt_bias, inp.A_log, inp.B, inp.C, inp.D, inp.z, inp.h0, ws)
