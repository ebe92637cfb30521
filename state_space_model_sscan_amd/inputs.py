"""Seeded synthetic inputs for the selective scan.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the scan's arithmetic. Both the CPU oracle and the HIP path
receive the very same arrays from here, so the oracle's fp64 run and the
GPU's run see identical bits.

Shapes follow the pages' served values:
  * Mamba-1 ("Mamba", nnterp guide, section "The values"): x, dt_raw, z are
    [batch, seq, channels]; B, C are [batch, seq, groups, state_dim]; the state
    is [batch, channels, state_dim]; A_log is [channels, state_dim].
  * Mamba-2 ("Mamba-2", nnterp encyclopedia, section "The mixer's values"):
    x, z are [batch, seq, heads, head_dim]; dt_raw is [batch, seq, heads];
    B, C are [batch, seq, groups, state_dim]; A_log, dt_bias, D are [heads].
    The state is stored [batch, heads, head_dim, state_dim].

Distributions (one stream per tensor, numpy PCG64 seeded from
SeedSequence([seed, tensor_id])):
  x, B, C, z ~ N(0, 1); dt_raw ~ N(0, 0.5^2);
  dt_bias = inverse-softplus of exp(u), u ~ U[ln 1e-3, ln 1e-1]
    (so the step at dt_raw = 0 lies in [1e-3, 1e-1], the usual init range);
  Mamba-1 A_log[c, n] = ln(n + 1); Mamba-2 A_log[h] = ln(U[1, 16]);
  D = 1 or D ~ U[0.5, 1.5]; h0 ~ N(0, 0.1^2).
Activations are drawn in float32 and rounded to bfloat16 (round to nearest
even) when the activation dtype is bf16. Parameters and states stay float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Fixed tensor ids for the per-tensor random streams.
TID = dict(x=0, dt_raw=1, dt_bias=2, B=3, C=4, z=5, D=6, h0=7, A_log=8,
           conv_w=9, conv_b=10, conv_state=11, norm_w=12)


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), TID[name]])))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    # keep NaN/inf patterns as they were (inf rounds to itself already)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _normal(seed, name, shape, std=1.0):
    g = _rng(seed, name)
    v = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


def _uniform(seed, name, shape, lo, hi):
    g = _rng(seed, name)
    return (lo + (hi - lo) * g.random(size=shape, dtype=np.float64))


def _dt_bias(seed, n):
    u = _uniform(seed, "dt_bias", (n,), math.log(1e-3), math.log(1e-1))
    # inverse softplus of exp(u): log(expm1(exp(u)))
    return np.log(np.expm1(np.exp(u))).astype(np.float32)


@dataclass
class Mamba1Inputs:
    batch: int
    seqlen: int
    channels: int
    state_dim: int
    ngroups: int
    act: str                 # "f32" or "bf16"
    bc_eps: float            # <= 0: no B/C RMS norm
    x: np.ndarray
    dt_raw: np.ndarray
    dt_bias: np.ndarray
    A_log: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: np.ndarray
    z: np.ndarray | None = None
    h0: np.ndarray | None = None
    want_states: bool = False
    meta: dict = field(default_factory=dict)


@dataclass
class SSDInputs:
    batch: int
    seqlen: int
    nheads: int
    head_dim: int
    state_dim: int
    ngroups: int
    chunk: int
    act: str
    x: np.ndarray
    dt_raw: np.ndarray
    dt_bias: np.ndarray
    A_log: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: np.ndarray
    z: np.ndarray | None = None
    h0: np.ndarray | None = None
    want_states: bool = False
    meta: dict = field(default_factory=dict)


def _act(a, act):
    return bf16_round(a) if act == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def make_mamba1(batch, seqlen, channels, state_dim=16, ngroups=1, act="f32", *, seed=0,
                gate=True, h0=False, D_mode="uniform", bc_eps=0.0, want_states=False,
                zero_step_frac=0.0, A_log_mode="arange") -> Mamba1Inputs:
    """Draw one Mamba-1 scan problem.

    zero_step_frac: fraction of (token, channel) entries whose dt_raw is -inf
    (a step of exactly zero). A_log_mode "arange" gives ln(n+1); "wide" draws
    ln|A| uniformly in [ln 4e-4, ln 36316], the span the Mamba-2 page reports for
    real weights; "random" draws ln(U[1, 16]) per entry.
    """
    L, Dc, N, G = seqlen, channels, state_dim, ngroups
    x = _act(_normal(seed, "x", (batch, L, Dc)), act)
    dt_raw = _normal(seed, "dt_raw", (batch, L, Dc), 0.5)
    if zero_step_frac > 0:
        m = _rng(seed + 1000, "dt_raw").random(size=dt_raw.shape) < zero_step_frac
        dt_raw[m] = -np.inf
    dt_raw = _act(dt_raw, act)
    B = _act(_normal(seed, "B", (batch, L, G, N)), act)
    C = _act(_normal(seed, "C", (batch, L, G, N)), act)
    dt_bias = _dt_bias(seed, Dc)
    if A_log_mode == "arange":
        A_log = np.broadcast_to(np.log(np.arange(1, N + 1, dtype=np.float64)), (Dc, N)).astype(np.float32)
    elif A_log_mode == "wide":
        A_log = _uniform(seed, "A_log", (Dc, N), math.log(4e-4), math.log(36316.0)).astype(np.float32)
    elif A_log_mode == "random":
        A_log = np.log(_uniform(seed, "A_log", (Dc, N), 1.0, 16.0)).astype(np.float32)
    else:
        raise ValueError(A_log_mode)
    A_log = np.ascontiguousarray(A_log)
    if D_mode == "ones":
        D = np.ones(Dc, np.float32)
    elif D_mode == "zeros":
        D = np.zeros(Dc, np.float32)
    else:
        D = _uniform(seed, "D", (Dc,), 0.5, 1.5).astype(np.float32)
    z = _act(_normal(seed, "z", (batch, L, Dc)), act) if gate else None
    hh = _normal(seed, "h0", (batch, Dc, N), 0.1) if h0 else None
    return Mamba1Inputs(batch, L, Dc, N, G, act, float(bc_eps), x, dt_raw, dt_bias, A_log, B, C, D,
                        z, hh, want_states)


def make_ssd(batch, seqlen, nheads, head_dim=64, state_dim=128, ngroups=1, act="bf16", *, seed=0,
             chunk=256, gate=True, h0=True, D_mode="uniform", want_states=False,
             zero_step_frac=0.0, A_log_mode="random") -> SSDInputs:
    """Draw one Mamba-2 (SSD) scan problem; A_log_mode "wide" spans [ln 4e-4, ln 36316]."""
    L, H, P, N, G = seqlen, nheads, head_dim, state_dim, ngroups
    x = _act(_normal(seed, "x", (batch, L, H, P)), act)
    dt_raw = _normal(seed, "dt_raw", (batch, L, H), 0.5)
    if zero_step_frac > 0:
        m = _rng(seed + 1000, "dt_raw").random(size=dt_raw.shape) < zero_step_frac
        dt_raw[m] = -np.inf
    dt_raw = _act(dt_raw, act)
    B = _act(_normal(seed, "B", (batch, L, G, N)), act)
    C = _act(_normal(seed, "C", (batch, L, G, N)), act)
    dt_bias = _dt_bias(seed, H)
    if A_log_mode == "random":
        A_log = np.log(_uniform(seed, "A_log", (H,), 1.0, 16.0)).astype(np.float32)
    elif A_log_mode == "wide":
        A_log = _uniform(seed, "A_log", (H,), math.log(4e-4), math.log(36316.0)).astype(np.float32)
    else:
        raise ValueError(A_log_mode)
    if D_mode == "ones":
        D = np.ones(H, np.float32)
    elif D_mode == "zeros":
        D = np.zeros(H, np.float32)
    else:
        D = _uniform(seed, "D", (H,), 0.5, 1.5).astype(np.float32)
    z = _act(_normal(seed, "z", (batch, L, H, P)), act) if gate else None
    hh = _normal(seed, "h0", (batch, H, P, N), 0.1) if h0 else None
    return SSDInputs(batch, L, H, P, N, G, chunk, act, x, dt_raw, dt_bias, A_log, B, C, D, z, hh,
                     want_states)


# The five workloads: shapes and distributions as the pages' model layers give them
# (Mamba-130m layer, Falcon-Mamba-7b width, Mamba-2 2.7B layer).
WORKLOADS = {
    0: dict(kind="mamba1", name="mamba1-fp32-1x64x1536-states", batch=1, seqlen=64, channels=1536,
            state_dim=16, act="f32", gate=False, h0=False, D_mode="ones", bc_eps=0.0, want_states=True),
    1: dict(kind="mamba1", name="mamba130m-layer-bf16-8x2048x1536", batch=8, seqlen=2048, channels=1536,
            state_dim=16, act="bf16", gate=True, h0=False, D_mode="uniform", bc_eps=0.0, want_states=False),
    2: dict(kind="mamba1", name="mamba1-fp32-decode-16x512x1536-h0", batch=16, seqlen=512, channels=1536,
            state_dim=16, act="f32", gate=True, h0=True, D_mode="uniform", bc_eps=0.0, want_states=False),
    3: dict(kind="mamba1", name="falcon-mamba7b-width-bf16-4x4096x8192-bcnorm", batch=4, seqlen=4096,
            channels=8192, state_dim=16, act="bf16", gate=True, h0=False, D_mode="uniform", bc_eps=1e-6,
            want_states=False),
    4: dict(kind="ssd", name="mamba2-2.7b-layer-bf16-4x8192x80x64-n128", batch=4, seqlen=8192, nheads=80,
            head_dim=64, state_dim=128, act="bf16", chunk=256, gate=True, h0=True, D_mode="uniform",
            want_states=False),
}


def make_workload(wid: int, seed: int | None = None, **overrides):
    """Inputs of workload `wid` (seed defaults to the workload id); overrides change sizes/options."""
    spec = dict(WORKLOADS[wid])
    spec.update(overrides)
    kind = spec.pop("kind")
    spec.pop("name")
    s = wid if seed is None else seed
    if kind == "mamba1":
        return make_mamba1(spec.pop("batch"), spec.pop("seqlen"), spec.pop("channels"), seed=s, **spec)
    return make_ssd(spec.pop("batch"), spec.pop("seqlen"), spec.pop("nheads"), seed=s, **spec)
