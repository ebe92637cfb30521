"""Thin ctypes binding of libsscan (include/sscan.h).

Argument marshalling only: shapes are read off the tensors to fill the
descriptor, outputs and the workspace are allocated with torch when the caller
does not pass them, device pointers and the current HIP stream are handed to
the C ABI, and a nonzero status raises SscanError. Every step of the scan runs
in libsscan's HIP kernels; if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsscan.so")

F32, BF16 = 0, 1
STATUS_NAMES = ["SSCAN_OK", "SSCAN_ERR_NULL", "SSCAN_ERR_SHAPE", "SSCAN_ERR_DTYPE", "SSCAN_ERR_UNSUPPORTED",
                "SSCAN_ERR_NOT_DEVICE", "SSCAN_ERR_ALIGN", "SSCAN_ERR_ALIAS", "SSCAN_ERR_WORKSPACE", "SSCAN_ERR_HIP"]
EXPORTS = ["sscan_mamba1_workspace_size", "sscan_mamba1_fwd", "sscan_step", "sscan_ssd_workspace_size",
           "sscan_ssd_fwd", "sscan_ssd_step", "sscan_ssd_attention_workspace_size", "sscan_ssd_attention", "sscan_conv1d_silu", "sscan_gated_rmsnorm",
           "sscan_status_string",
           "sscan_last_error", "sscan_abi_version", "sscan_set_pointer_checks", "sscan_set_tuning",
           "sscan_ssd_fwd_noalloc"]

# Knobs of sscan_set_tuning (include/sscan.h).
TUNE_M1_LANES, TUNE_SSD_SEGMENT_CHUNKS, TUNE_SSD_WORKGROUPS, TUNE_SSD_GIVE_UP = 1, 2, 3, 4
TUNE_SSD_HEADS_PER_WORKGROUP = 5
TUNE_SSD_F32_TOKEN_LOOP = 6
TUNE_SSD_TWO_PASS = 7
TUNE_SSD_SPLIT_STATE = 8
# Byte offset of the give-up word in the workspace of an SSD call on the MFMA chunk path.
SSD_GIVEUP_WORD_OFFSET = 512


class Mamba1Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("channels", ctypes.c_int64),
                ("state_dim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("act", ctypes.c_int32),
                ("bc_rms_eps", ctypes.c_float)]


class SSDDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("state_dim", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("act", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ConvDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("channels", ctypes.c_int64),
                ("width", ctypes.c_int64), ("act", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SscanError(RuntimeError):
    def __init__(self, status: int, detail: str):
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__("%s: %s" % (name, detail))
        self.status = status
        self.name = name
        self.detail = detail


_lib = None


def lib():
    """The loaded libsscan (ctypes.CDLL) with argument types set. Raises if not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libsscan.so is not built at %s; run __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    M1 = ctypes.POINTER(Mamba1Desc)
    SD = ctypes.POINTER(SSDDesc)
    L.sscan_mamba1_workspace_size.argtypes = [M1]
    L.sscan_mamba1_workspace_size.restype = S
    L.sscan_mamba1_fwd.argtypes = [M1] + [P] * 13 + [S, P]
    L.sscan_mamba1_fwd.restype = I
    L.sscan_step.argtypes = [M1] + [P] * 12
    L.sscan_step.restype = I
    L.sscan_ssd_workspace_size.argtypes = [SD]
    L.sscan_ssd_workspace_size.restype = S
    L.sscan_ssd_fwd.argtypes = [SD] + [P] * 13 + [S, P]
    L.sscan_ssd_fwd.restype = I
    L.sscan_ssd_fwd_noalloc.argtypes = [SD] + [P] * 13
    L.sscan_ssd_fwd_noalloc.restype = I
    L.sscan_ssd_step.argtypes = [SD] + [P] * 12
    L.sscan_ssd_step.restype = I
    L.sscan_ssd_attention_workspace_size.argtypes = [SD]
    L.sscan_ssd_attention_workspace_size.restype = S
    L.sscan_ssd_attention.argtypes = [SD] + [P] * 7 + [S, P]
    L.sscan_ssd_attention.restype = I
    L.sscan_conv1d_silu.argtypes = [ctypes.POINTER(ConvDesc)] + [P] * 7
    L.sscan_conv1d_silu.restype = I
    L.sscan_gated_rmsnorm.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, P, P, P, ctypes.c_float, P, P]
    L.sscan_gated_rmsnorm.restype = I
    L.sscan_status_string.argtypes = [I]
    L.sscan_status_string.restype = ctypes.c_char_p
    L.sscan_last_error.argtypes = []
    L.sscan_last_error.restype = ctypes.c_char_p
    L.sscan_abi_version.argtypes = []
    L.sscan_abi_version.restype = I
    L.sscan_set_pointer_checks.argtypes = [I]
    L.sscan_set_pointer_checks.restype = I
    L.sscan_set_tuning.argtypes = [I, ctypes.c_int64]
    L.sscan_set_tuning.restype = ctypes.c_int64
    _lib = L
    return L


def check(status: int):
    if status != 0:
        raise SscanError(status, lib().sscan_last_error().decode())


def set_pointer_checks(enabled: bool) -> bool:
    return bool(lib().sscan_set_pointer_checks(1 if enabled else 0))


def set_tuning(knob: int, value: int) -> int:
    """Set a process-wide launch-plan override (0: the library's choice); returns the previous value."""
    prev = int(lib().sscan_set_tuning(int(knob), int(value)))
    if prev < 0:
        raise ValueError("unknown tuning knob %r or negative value %r" % (knob, value))
    return prev


def _shape(name, t, shape):
    """The C ABI cannot see buffer sizes: every tensor's shape is checked here, before the call."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


def _act_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("activations must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libsscan takes contiguous tensors")
    return t.data_ptr()


def _f32(name, t):
    if t is not None and t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    return t


def _same(name, t, dtype):
    if t is not None and t.dtype != dtype:
        raise TypeError("%s must be %s like x, got %s" % (name, dtype, t.dtype))
    return t


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream().cuda_stream


def mamba1_desc(x, B, bc_rms_eps=0.0):
    b, L, Dc = x.shape
    G, N = B.shape[2], B.shape[3]
    return Mamba1Desc(b, L, Dc, N, G, _act_code(x), float(bc_rms_eps))


def ssd_desc(x, B, chunk=0):
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return SSDDesc(b, L, H, P, N, G, int(chunk), _act_code(x), 0)


def sscan_mamba1_workspace_size(desc: Mamba1Desc) -> int:
    return int(lib().sscan_mamba1_workspace_size(ctypes.byref(desc)))


def sscan_ssd_workspace_size(desc: SSDDesc) -> int:
    return int(lib().sscan_ssd_workspace_size(ctypes.byref(desc)))


def _check_mamba1(b, L, Dc, N, G, x, dt_raw, dt_bias, A_log, B, C, D, z, state_input, y, state_output):
    for n, t, sh in (("dt_raw", dt_raw, (b, L, Dc)), ("dt_bias", dt_bias, (Dc,)), ("A_log", A_log, (Dc, N)),
                     ("B", B, (b, L, G, N)), ("C", C, (b, L, G, N)), ("D", D, (Dc,)), ("z", z, (b, L, Dc)),
                     ("state_input", state_input, (b, Dc, N)), ("y", y, (b, L, Dc)),
                     ("state_output", state_output, (b, Dc, N))):
        _shape(n, t, sh)
    _same("y", y, x.dtype)
    _f32("state_output", state_output)


def _check_ssd(b, L, H, P, N, G, x, dt_raw, dt_bias, A_log, B, C, D, z, state_input, y, state_output):
    for n, t, sh in (("dt_raw", dt_raw, (b, L, H)), ("dt_bias", dt_bias, (H,)), ("A_log", A_log, (H,)),
                     ("B", B, (b, L, G, N)), ("C", C, (b, L, G, N)), ("D", D, (H,)), ("z", z, (b, L, H, P)),
                     ("state_input", state_input, (b, H, P, N)), ("y", y, (b, L, H, P)),
                     ("state_output", state_output, (b, H, P, N))):
        _shape(n, t, sh)
    _same("y", y, x.dtype)
    _f32("state_output", state_output)


def _workspace_bytes(workspace):
    return workspace.numel() * workspace.element_size() if workspace is not None else 0


def sscan_mamba1_fwd(x, dt_raw, dt_bias, A_log, B, C, D, z=None, state_input=None, y=None,
                     state_output=None, states=None, workspace=None, bc_rms_eps=0.0, want_states=False,
                     stream=None):
    """Mamba-1 scan over a prompt. x, dt_raw, z: [b, L, Dc]; B, C: [b, L, G, N].
    Returns (y, state_output, states or None)."""
    desc = mamba1_desc(x, B, bc_rms_eps)
    for n, t in (("dt_raw", dt_raw), ("B", B), ("C", C), ("z", z)):
        _same(n, t, x.dtype)
    for n, t in (("dt_bias", dt_bias), ("A_log", A_log), ("D", D), ("state_input", state_input)):
        _f32(n, t)
    b, L, Dc = x.shape
    G, N = B.shape[2], B.shape[3]
    _check_mamba1(b, L, Dc, N, G, x, dt_raw, dt_bias, A_log, B, C, D, z, state_input, y, state_output)
    _shape("states", states, (b, L, Dc, N))
    _f32("states", states)
    if y is None:
        y = torch.empty_like(x)
    if state_output is None:
        state_output = torch.empty((b, Dc, N), dtype=torch.float32, device=x.device)
    if states is None and want_states:
        states = torch.empty((b, L, Dc, N), dtype=torch.float32, device=x.device)
    ws_bytes = sscan_mamba1_workspace_size(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    wb = _workspace_bytes(workspace)
    check(lib().sscan_mamba1_fwd(ctypes.byref(desc), _ptr(x), _ptr(dt_raw), _ptr(dt_bias), _ptr(A_log), _ptr(B),
                                 _ptr(C), _ptr(D), _ptr(z), _ptr(state_input), _ptr(y), _ptr(state_output),
                                 _ptr(states), _ptr(workspace), wb, _stream(stream)))
    return y, state_output, states


def sscan_step(state_input, x, dt_raw, dt_bias, A_log, B, C, D, z=None, y=None, state_output=None,
               bc_rms_eps=0.0, stream=None):
    """Mamba-1 one-token decode step. x, dt_raw, z: [b, 1, Dc]; B, C: [b, 1, G, N]; state [b, Dc, N].
    state_output may be state_input (in place). Returns (y, state_output)."""
    desc = mamba1_desc(x, B, bc_rms_eps)
    for n, t in (("dt_raw", dt_raw), ("B", B), ("C", C), ("z", z)):
        _same(n, t, x.dtype)
    for n, t in (("dt_bias", dt_bias), ("A_log", A_log), ("D", D), ("state_input", state_input)):
        _f32(n, t)
    if state_input is None:
        raise ValueError("sscan_step needs state_input")
    b, L, Dc = x.shape
    if L != 1:
        raise ValueError("sscan_step takes one token: x must be [b, 1, channels]")
    _check_mamba1(b, 1, Dc, B.shape[3], B.shape[2], x, dt_raw, dt_bias, A_log, B, C, D, z, state_input, y,
                  state_output)
    if y is None:
        y = torch.empty_like(x)
    if state_output is None:
        state_output = torch.empty_like(state_input)
    check(lib().sscan_step(ctypes.byref(desc), _ptr(state_input), _ptr(state_output), _ptr(x), _ptr(dt_raw),
                           _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y),
                           _stream(stream)))
    return y, state_output


def sscan_ssd_fwd(x, dt_raw, dt_bias, A_log, B, C, D, z=None, state_input=None, y=None, state_output=None,
                  states=None, workspace=None, chunk=0, want_states=False, stream=None):
    """Mamba-2 SSD over a prompt. x, z: [b, L, H, P]; dt_raw: [b, L, H]; B, C: [b, L, G, N].
    Returns (y, state_output [b, H, P, N], states [b, L, H, P, N] or None)."""
    desc = ssd_desc(x, B, chunk)
    for n, t in (("dt_raw", dt_raw), ("B", B), ("C", C), ("z", z)):
        _same(n, t, x.dtype)
    for n, t in (("dt_bias", dt_bias), ("A_log", A_log), ("D", D), ("state_input", state_input)):
        _f32(n, t)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _check_ssd(b, L, H, P, N, G, x, dt_raw, dt_bias, A_log, B, C, D, z, state_input, y, state_output)
    _shape("states", states, (b, L, H, P, N))
    _f32("states", states)
    if y is None:
        y = torch.empty_like(x)
    if state_output is None:
        state_output = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    if states is None and want_states:
        states = torch.empty((b, L, H, P, N), dtype=torch.float32, device=x.device)
    ws_bytes = sscan_ssd_workspace_size(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    wb = _workspace_bytes(workspace)
    check(lib().sscan_ssd_fwd(ctypes.byref(desc), _ptr(x), _ptr(dt_raw), _ptr(dt_bias), _ptr(A_log), _ptr(B),
                              _ptr(C), _ptr(D), _ptr(z), _ptr(state_input), _ptr(y), _ptr(state_output),
                              _ptr(states), _ptr(workspace), wb, _stream(stream)))
    return y, state_output, states


def sscan_ssd_fwd_noalloc(x, dt_raw, dt_bias, A_log, B, C, D, z=None, state_input=None, y=None,
                          state_output=None, states=None, chunk=0, stream=None):
    """sscan_ssd_fwd without a workspace: the library's static device scratch takes its
    place (for callers that cannot allocate). Outputs are allocated here when not given.
    Returns (y, state_output, states or None)."""
    desc = ssd_desc(x, B, chunk)
    for n, t in (("dt_raw", dt_raw), ("B", B), ("C", C), ("z", z)):
        _same(n, t, x.dtype)
    for n, t in (("dt_bias", dt_bias), ("A_log", A_log), ("D", D), ("state_input", state_input)):
        _f32(n, t)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _check_ssd(b, L, H, P, N, G, x, dt_raw, dt_bias, A_log, B, C, D, z, state_input, y, state_output)
    _shape("states", states, (b, L, H, P, N))
    _f32("states", states)
    if y is None:
        y = torch.empty_like(x)
    if state_output is None:
        state_output = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    check(lib().sscan_ssd_fwd_noalloc(ctypes.byref(desc), _ptr(x), _ptr(dt_raw), _ptr(dt_bias), _ptr(A_log),
                                      _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(state_input), _ptr(y),
                                      _ptr(state_output), _ptr(states), _stream(stream)))
    return y, state_output, states


def sscan_ssd_step(state_input, x, dt_raw, dt_bias, A_log, B, C, D, z=None, y=None, state_output=None,
                   stream=None):
    """Mamba-2 one-token decode step. x, z: [b, 1, H, P]; dt_raw [b, 1, H]; state [b, H, P, N]."""
    desc = ssd_desc(x, B, 0)
    for n, t in (("dt_raw", dt_raw), ("B", B), ("C", C), ("z", z)):
        _same(n, t, x.dtype)
    for n, t in (("dt_bias", dt_bias), ("A_log", A_log), ("D", D), ("state_input", state_input)):
        _f32(n, t)
    if state_input is None:
        raise ValueError("sscan_ssd_step needs state_input")
    b, L, H, P = x.shape
    if L != 1:
        raise ValueError("sscan_ssd_step takes one token: x must be [b, 1, heads, head_dim]")
    _check_ssd(b, 1, H, P, B.shape[3], B.shape[2], x, dt_raw, dt_bias, A_log, B, C, D, z, state_input, y,
               state_output)
    if y is None:
        y = torch.empty_like(x)
    if state_output is None:
        state_output = torch.empty_like(state_input)
    check(lib().sscan_ssd_step(ctypes.byref(desc), _ptr(state_input), _ptr(state_output), _ptr(x), _ptr(dt_raw),
                               _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y),
                               _stream(stream)))
    return y, state_output


def sscan_ssd_attention(dt_raw, dt_bias, A_log, B, C, alpha=None, workspace=None, stream=None):
    """The SSD scan's hidden attention map. dt_raw: [b, L, H]; B, C: [b, L, G, N] (same dtype).
    Returns alpha [b, L (query), L (key), H] f32: y_t = sum_s alpha[t, s] x_s + D x_t before the gate.
    The workspace (b * L * H * 12 bytes) is allocated here when not given."""
    _same("B", B, dt_raw.dtype)
    _same("C", C, dt_raw.dtype)
    for n, t in (("dt_bias", dt_bias), ("A_log", A_log)):
        _f32(n, t)
    b, L, H = dt_raw.shape
    G, N = B.shape[2], B.shape[3]
    for n, t, sh in (("dt_bias", dt_bias, (H,)), ("A_log", A_log, (H,)), ("B", B, (b, L, G, N)),
                     ("C", C, (b, L, G, N)), ("alpha", alpha, (b, L, L, H))):
        _shape(n, t, sh)
    _f32("alpha", alpha)
    desc = SSDDesc(b, L, H, 1, N, G, 0, _act_code(dt_raw), 0)
    if alpha is None:
        alpha = torch.empty((b, L, L, H), dtype=torch.float32, device=dt_raw.device)
    need = int(lib().sscan_ssd_attention_workspace_size(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dt_raw.device)
    wb = workspace.numel() * workspace.element_size()
    check(lib().sscan_ssd_attention(ctypes.byref(desc), _ptr(dt_raw), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C),
                                    _ptr(alpha), _ptr(workspace), wb, _stream(stream)))
    return alpha


def sscan_conv1d_silu(x, weight, bias=None, conv_state_in=None, out=None, conv_state_out=None,
                      want_state=True, stream=None):
    """Causal depthwise conv1d + silu. x: [b, L, Dc] (f32/bf16); weight: [Dc, W] f32;
    conv state [b, Dc, W-1] f32. Returns (out, conv_state_out or None)."""
    b, L, Dc = x.shape
    W = weight.shape[1]
    for n, t in (("weight", weight), ("bias", bias), ("conv_state_in", conv_state_in),
                 ("conv_state_out", conv_state_out)):
        _f32(n, t)
    for n, t, sh in (("weight", weight, (Dc, W)), ("bias", bias, (Dc,)), ("conv_state_in", conv_state_in,
                     (b, Dc, W - 1)), ("out", out, (b, L, Dc)), ("conv_state_out", conv_state_out, (b, Dc, W - 1))):
        _shape(n, t, sh)
    _same("out", out, x.dtype)
    desc = ConvDesc(b, L, Dc, W, _act_code(x), 0)
    if out is None:
        out = torch.empty_like(x)
    if conv_state_out is None and want_state and W > 1:
        conv_state_out = torch.empty((b, Dc, W - 1), dtype=torch.float32, device=x.device)
    check(lib().sscan_conv1d_silu(ctypes.byref(desc), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state_in),
                                  _ptr(out), _ptr(conv_state_out), _stream(stream)))
    return out, conv_state_out


def sscan_gated_rmsnorm(y, z, weight, eps, out=None, stream=None):
    """out = (y * silu(z)) / sqrt(mean over the last axis + eps) * weight. y, z: [..., width]."""
    _same("z", z, y.dtype)
    _same("out", out, y.dtype)
    _f32("weight", weight)
    _shape("z", z, y.shape)
    _shape("out", out, y.shape)
    _shape("weight", weight, (y.shape[-1],))
    width = y.shape[-1]
    rows = y.numel() // width if width else 0
    if out is None:
        out = torch.empty_like(y)
    check(lib().sscan_gated_rmsnorm(rows, width, _act_code(y), _ptr(y), _ptr(z), _ptr(weight), float(eps), _ptr(out),
                                    _stream(stream)))
    return out


def ssd_state_key_first(state: torch.Tensor) -> torch.Tensor:
    """The pages' [b, H, key (state_dim), value (head_dim)] view of a [b, H, P, N] state."""
    return state.transpose(-1, -2)
