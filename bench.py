"""Benchmark of the selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only-main]

A step is one sscan_mamba1_fwd over the Mamba-130m layer workload (batch 8,
seq 2048, d_inner 1536, state_dim 16, bf16 activations, fp32 state, fused
silu(z) gate). Inputs are resident in HBM when timing starts; three copies of
them rotate so no step finds its inputs in the 256 MiB Infinity Cache. K steps
are timed between two device synchronizations; each call is also bracketed by
HIP events on the stream the kernels are launched on. Beside the main line the
run reports the Falcon-Mamba-7b-width Mamba-1 workload, the Mamba-2 2.7B SSD
workload, the 512-call decode-step workload, the Mamba-2 decode step, the
conv1d + silu and gated RMS norm around the Mamba-2 scan, the hidden attention
map, the SSD with per-token states, and the fp64 CPU oracle timed on this host.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, published
# VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (one fp32 op per lane per
# slot; v_exp_f32 takes two slots). Peak in T lane-slots/s.
VALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12
METRIC = "scan tokens/s & % HBM roofline (Mamba-1); SSD tokens/s & % MFMA peak"
MAIN_KERNEL = "m1_row_kernel<bf16, 16 states, gate> (a 16-lane row per channel)"
# sources of the main kernel: HBM traffic from hardware counters is reported only
# while these hash to the value recorded with the counters
MAIN_KERNEL_SOURCES = ["state_space_model_sscan_amd/csrc/m1_row_impl.hpp",
                       "state_space_model_sscan_amd/csrc/m1_fast_impl.hpp",
                       "state_space_model_sscan_amd/csrc/m1_fast.hip",
                       "state_space_model_sscan_amd/csrc/m1r_bf16_16.hip",
                       "state_space_model_sscan_amd/csrc/device_common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")


def sources_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_key):
    """HBM bytes per launch measured by FETCH_SIZE/WRITE_SIZE (scaled by a plain copy's
    reading), from the counter summary in profiles/, if it is for the current source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get(kernel_key)
    if not rec or rec.get("sources_sha256_16") != sources_hash(rec.get("sources", [])):
        return None
    return rec


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def upload(inp, torch):
    def act(a):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
        return (t.to(torch.bfloat16) if inp.act == "bf16" else t).cuda()

    def par(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()

    return dict(x=act(inp.x), dt_raw=act(inp.dt_raw), B=act(inp.B), C=act(inp.C), z=act(inp.z),
                dt_bias=par(inp.dt_bias), A_log=par(inp.A_log), D=par(inp.D), state_input=par(inp.h0))


def clone_set(d):
    return {k: (None if v is None else v.clone()) for k, v in d.items()}


def mamba1_bytes(inp):
    b, L, Dc, N, G = inp.batch, inp.seqlen, inp.channels, inp.state_dim, inp.ngroups
    es = 2 if inp.act == "bf16" else 4
    nact = 3 if inp.z is not None else 2
    rd = nact * b * L * Dc * es + 2 * b * L * G * N * es + (2 * Dc + Dc * N) * 4
    if inp.h0 is not None:
        rd += b * Dc * N * 4
    wr = b * L * Dc * es + b * Dc * N * 4
    return rd + wr


def ssd_bytes(inp):
    b, L, H, P, N, G = inp.batch, inp.seqlen, inp.nheads, inp.head_dim, inp.state_dim, inp.ngroups
    es = 2 if inp.act == "bf16" else 4
    nact = 2 if inp.z is not None else 1
    rd = nact * b * L * H * P * es + b * L * H * es + 2 * b * L * G * N * es + 3 * H * 4
    if inp.h0 is not None:
        rd += b * H * P * N * 4
    wr = b * L * H * P * es + b * H * P * N * 4
    return rd + wr


def ssd_flops(inp, Q=256):
    """Contraction FLOPs of the chunked SSD at chunk Q (dense Q x Q blocks): C.B^T per
    (batch, chunk, group), and per (batch, chunk, head) the diagonal block M.X, the chunk
    state X^T.(B*w) and the off-diagonal read C.H^T."""
    b, L, H, P, N, G = inp.batch, inp.seqlen, inp.nheads, inp.head_dim, inp.state_dim, inp.ngroups
    nch = -(-L // Q)
    return b * nch * (G * 2 * Q * Q * N + H * (2 * Q * Q * P + 2 * Q * N * P + 2 * Q * N * P))


def time_calls(fn, sets, steps, warmup, torch):
    """Run fn(set) `warmup` times untimed, then `steps` times timed; returns
    (wall ms per step, mean event ms per call)."""
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        fn(sets[i % len(sets)])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    return wall, ev


def bench_mamba1(wid, steps, warmup, torch, bd, gen):
    inp = gen.make_workload(wid)
    base = upload(inp, torch)
    sets = [base] + [clone_set(base) for _ in range(2)]
    b, L, Dc, N = inp.batch, inp.seqlen, inp.channels, inp.state_dim
    y = torch.empty_like(base["x"])
    h = torch.empty((b, Dc, N), dtype=torch.float32, device="cuda")
    ws_n = bd.sscan_mamba1_workspace_size(bd.mamba1_desc(base["x"], base["B"], inp.bc_eps))
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def fn(s):
        bd.sscan_mamba1_fwd(s["x"], s["dt_raw"], s["dt_bias"], s["A_log"], s["B"], s["C"], s["D"], s["z"],
                            s["state_input"], y=y, state_output=h, workspace=ws, bc_rms_eps=inp.bc_eps)

    wall, ev = time_calls(fn, sets, steps, warmup, torch)
    upd = b * L * Dc * N
    by = mamba1_bytes(inp)
    return dict(workload=gen.WORKLOADS[wid]["name"], ms_per_step=wall, kernel_ms=ev, tokens=b * L,
                tokens_per_s=b * L / (wall * 1e-3), updates_per_s=upd / (ev * 1e-3), bytes=by,
                hbm_gbs=by / (ev * 1e-3) / 1e9, hbm_frac=by / (ev * 1e-3) / 1e9 / HBM_PEAK_GBS,
                valu_tslots=6 * upd / (ev * 1e-3) / 1e12, inp=inp)


def bench_ssd(steps, warmup, torch, bd, gen):
    inp = gen.make_workload(4)
    base = upload(inp, torch)
    sets = [base] + [clone_set(base) for _ in range(2)]
    b, L, H, P, N = inp.batch, inp.seqlen, inp.nheads, inp.head_dim, inp.state_dim
    y = torch.empty_like(base["x"])
    h = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    ws_n = bd.sscan_ssd_workspace_size(bd.ssd_desc(base["x"], base["B"], inp.chunk))
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def fn(s):
        bd.sscan_ssd_fwd(s["x"], s["dt_raw"], s["dt_bias"], s["A_log"], s["B"], s["C"], s["D"], s["z"],
                         s["state_input"], y=y, state_output=h, workspace=ws, chunk=inp.chunk)

    wall, ev = time_calls(fn, sets, steps, warmup, torch)
    by = ssd_bytes(inp)
    fl = ssd_flops(inp, 256)
    return dict(workload=gen.WORKLOADS[4]["name"], ms_per_step=wall, kernel_ms=ev, tokens=b * L,
                tokens_per_s=b * L / (wall * 1e-3), bytes=by, hbm_gbs=by / (ev * 1e-3) / 1e9,
                hbm_frac=by / (ev * 1e-3) / 1e9 / HBM_PEAK_GBS, flops_q256=fl,
                mfma_tflops=fl / (ev * 1e-3) / 1e12, mfma_frac=fl / (ev * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                inp=inp, base=base)


def bench_step(torch, bd, gen, calls=512):
    """Workload 2 as `calls` one-token sscan_step calls, state updated in place: timed
    eagerly (includes the Python/ctypes cost of each call) and as a HIP graph that
    replays the same `calls` launches (the GPU-side cost per step)."""
    inp = gen.make_workload(2)
    base = upload(inp, torch)
    b, Dc = inp.batch, inp.channels
    xs = [base["x"][:, t:t + 1].contiguous() for t in range(calls)]
    dts = [base["dt_raw"][:, t:t + 1].contiguous() for t in range(calls)]
    zs = [base["z"][:, t:t + 1].contiguous() for t in range(calls)]
    Bs = [base["B"][:, t:t + 1].contiguous() for t in range(calls)]
    Cs = [base["C"][:, t:t + 1].contiguous() for t in range(calls)]
    state = base["state_input"].clone()
    ys = [torch.empty_like(xs[0]) for _ in range(calls)]

    def run(n):
        for t in range(n):
            bd.sscan_step(state, xs[t], dts[t], base["dt_bias"], base["A_log"], Bs[t], Cs[t], base["D"], zs[t],
                          y=ys[t], state_output=state)

    run(8)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    run(calls)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e6 / calls
    eager_gpu = e0.elapsed_time(e1) * 1e3 / calls
    # the same calls captured once into a HIP graph (pointer checks are host-side queries:
    # off while capturing), then replayed
    graph_us = None
    try:
        prev = bd.set_pointer_checks(False)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(calls)
        bd.set_pointer_checks(prev)
        g.replay()
        torch.cuda.synchronize()
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / (reps * calls)
    except Exception as ex:  # report, do not fail the bench
        log("graph capture of the decode steps failed: %s" % ex)
    per_call_bytes = 2 * b * Dc * 16 * 4 + 4 * b * Dc * 4 + 2 * b * 16 * 4 + (2 * Dc + Dc * 16) * 4
    return dict(workload=gen.WORKLOADS[2]["name"] + " as %d sscan_step calls" % calls,
                us_per_step_wall=wall, us_per_step_gpu_eager=eager_gpu, us_per_step_graph=graph_us,
                bytes_per_call=per_call_bytes,
                graph_gbs=None if not graph_us else per_call_bytes / (graph_us * 1e-6) / 1e9)


def hbm_entry(workload, ms_wall, ms_kernel, nbytes, **kw):
    d = dict(workload=workload, ms_per_step=ms_wall, kernel_ms=ms_kernel, bytes=nbytes,
             hbm_gbs=nbytes / (ms_kernel * 1e-3) / 1e9, hbm_frac=nbytes / (ms_kernel * 1e-3) / 1e9 / HBM_PEAK_GBS)
    d.update(kw)
    return d


def bench_mixer_ops(steps, warmup, torch, bd, s4):
    """The steps next to the scan at the Mamba-2 2.7B layer shape (batch 4, 8192 tokens):
    conv1d + silu over xBC (5120 + 2 x 128 = 5376 channels, width 4, with the carried conv
    state in and out), and the gated RMS norm over y, z (80 heads x 64 = 5120 wide). Both
    stream more than the 256 MiB Infinity Cache per call."""
    base = s4["base"]
    b, L = base["x"].shape[0], base["x"].shape[1]
    g = torch.Generator(device="cuda")
    g.manual_seed(5376)
    Dc, W = 5376, 4
    xbc = torch.randn((b, L, Dc), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((Dc, W), generator=g, device="cuda") * 0.5).contiguous()
    bias = torch.randn((Dc,), generator=g, device="cuda") * 0.1
    cst = torch.randn((b, Dc, W - 1), generator=g, device="cuda")
    out = torch.empty_like(xbc)
    cst_out = torch.empty_like(cst)

    def conv(_):
        bd.sscan_conv1d_silu(xbc, w, bias, cst, out=out, conv_state_out=cst_out)

    wall, ev = time_calls(conv, [None], steps, warmup, torch)
    cbytes = 2 * b * L * Dc * 2 + Dc * (W + 1) * 4 + 2 * b * Dc * (W - 1) * 4
    conv_e = hbm_entry("mamba2-2.7b xBC conv1d+silu, bf16 %dx%dx%d, width %d, conv state in/out" % (b, L, Dc, W),
                       wall, ev, cbytes, tokens_per_s=b * L / (wall * 1e-3))
    del xbc, out

    rows, width = b * L, base["x"].shape[2] * base["x"].shape[3]
    y2, z2 = base["x"].view(rows, width), base["z"].view(rows, width)
    wn = torch.rand((width,), generator=g, device="cuda") + 0.5
    nout = torch.empty_like(y2)

    def norm(_):
        bd.sscan_gated_rmsnorm(y2, z2, wn, 1e-5, out=nout)

    wall, ev = time_calls(norm, [None], steps, warmup, torch)
    nbytes = 3 * rows * width * 2 + width * 4
    norm_e = hbm_entry("mamba2-2.7b gated RMS norm, bf16 %d rows x %d" % (rows, width), wall, ev, nbytes,
                       tokens_per_s=rows / (wall * 1e-3))
    return conv_e, norm_e


def bench_ssd_step(torch, bd, s4, nstates=32, calls=64):
    """Mamba-2 2.7B decode: one-token sscan_ssd_step calls at batch 4 (state [4, 80, 64, 128]
    fp32, 10.5 MB, updated in place). The calls cycle over `nstates` separate states, 336 MB
    in all, so that no call finds its state in the 256 MiB Infinity Cache, as in a model whose
    other layers' states pass through between two steps of a layer. Timed as a HIP graph
    that replays `calls` launches."""
    base = s4["base"]
    one = lambda a, t: a[:, t:t + 1].contiguous()
    xs = [one(base["x"], t) for t in range(calls)]
    zs = [one(base["z"], t) for t in range(calls)]
    dts = [one(base["dt_raw"], t) for t in range(calls)]
    Bs = [one(base["B"], t) for t in range(calls)]
    Cs = [one(base["C"], t) for t in range(calls)]
    ys = [torch.empty_like(xs[0]) for _ in range(calls)]
    states = [base["state_input"].clone() for _ in range(nstates)]

    def run():
        for t in range(calls):
            st = states[t % nstates]
            bd.sscan_ssd_step(st, xs[t], dts[t], base["dt_bias"], base["A_log"], Bs[t], Cs[t], base["D"], zs[t],
                              y=ys[t], state_output=st)

    run()
    torch.cuda.synchronize()
    prev = bd.set_pointer_checks(False)
    try:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            run()
    finally:
        bd.set_pointer_checks(prev)
    gr.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        gr.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * calls)
    bsz, _, H, P = xs[0].shape
    N = Bs[0].shape[-1]
    G = Bs[0].shape[2]
    per_call = 2 * bsz * H * P * N * 4 + 3 * bsz * H * P * 2 + bsz * H * 2 + 2 * bsz * G * N * 2 + 3 * H * 4
    return dict(workload="mamba2-2.7b decode: sscan_ssd_step, batch %d, %d heads x %d, state %d, fp32 state "
                         "in place, %d states in rotation" % (bsz, H, P, N, nstates),
                us_per_step_graph=us, bytes_per_call=per_call, hbm_gbs=per_call / (us * 1e-6) / 1e9,
                hbm_frac=per_call / (us * 1e-6) / 1e9 / HBM_PEAK_GBS)


def bench_ssd_states(steps, warmup, torch, bd, gen):
    """sscan_ssd_fwd with per-token states at the Mamba2-130m mixer shape (24 heads x 64,
    state 128, bf16) over one sequence of 512 tokens: the states [1, 512, 24, 64, 128] fp32
    (403 MB) are the output that dominates."""
    inp = gen.make_ssd(1, 512, 24, 64, 128, act="bf16", seed=130, gate=True, h0=True, want_states=True)
    base = upload(inp, torch)
    b, L, H, P, N = inp.batch, inp.seqlen, inp.nheads, inp.head_dim, inp.state_dim
    y = torch.empty_like(base["x"])
    h = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    states = torch.empty((b, L, H, P, N), dtype=torch.float32, device="cuda")
    ws_n = bd.sscan_ssd_workspace_size(bd.ssd_desc(base["x"], base["B"], inp.chunk))
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def fn(_):
        bd.sscan_ssd_fwd(base["x"], base["dt_raw"], base["dt_bias"], base["A_log"], base["B"], base["C"], base["D"],
                         base["z"], base["state_input"], y=y, state_output=h, states=states, workspace=ws,
                         chunk=inp.chunk)

    wall, ev = time_calls(fn, [None], steps, warmup, torch)
    nbytes = ssd_bytes(inp) + b * L * H * P * N * 4
    return hbm_entry("mamba2-130m mixer with per-token states, bf16 1x512 tokens x 24 heads x 64, state 128",
                     wall, ev, nbytes, tokens_per_s=b * L / (wall * 1e-3))


def bench_attention(steps, warmup, torch, bd, s4, L=2048):
    """The hidden attention map of batch row 0's first L tokens of the Mamba-2 2.7B workload
    (80 heads, one group, state 128): alpha [1, L, L, 80] fp32, 1.34 GB written per call."""
    base = s4["base"]
    dt = base["dt_raw"][:1, :L].contiguous()
    B = base["B"][:1, :L].contiguous()
    C = base["C"][:1, :L].contiguous()
    H = dt.shape[2]
    alpha = torch.empty((1, L, L, H), dtype=torch.float32, device="cuda")

    def fn(_):
        bd.sscan_ssd_attention(dt, base["dt_bias"], base["A_log"], B, C, alpha=alpha)

    wall, ev = time_calls(fn, [None], steps, warmup, torch)
    nbytes = L * L * H * 4 + L * H * 2 + 2 * L * B.shape[2] * B.shape[3] * 2 + 2 * H * 4
    return hbm_entry("mamba2-2.7b hidden attention map, 1 x %d tokens x %d heads, fp32 out" % (L, H), wall, ev,
                     nbytes)


def cpu_baseline(inp, min_seconds=10.0, max_runs=200):
    """The fp64 oracle on the same workload, run whole and repeated until at least
    `min_seconds` of CPU work have been timed; reports the mean rate over the runs."""
    import oracle

    oracle.build(force=False)
    runs, total = 0, 0.0
    while runs < 2 or (total < min_seconds and runs < max_runs):
        t0 = time.perf_counter()
        oracle.run_inputs(inp, want_states=False)
        total += time.perf_counter() - t0
        runs += 1
    toks = inp.batch * inp.seqlen * runs
    return dict(value=toks / total, unit="tokens/s", cores=oracle.threads(), kind="oracle",
                sample="the whole workload (%d x %d tokens x %d channels x %d states), fp64, run %d times "
                       "back to back, %.1f s in all" % (inp.batch, inp.seqlen, inp.channels, inp.state_dim, runs,
                                                        total))


def copy_calibration(torch, gib=1, reps=3):
    """A plain elementwise kernel of known traffic (reads 1 GiB, writes 1 GiB), for
    scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = gib * (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        torch.add(a, 1.0, out=b)
    torch.cuda.synchronize()
    log("copy calibration: %d x elementwise copy of %d bytes" % (reps, n * 4))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-main", action="store_true", help="time only the main workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (every box has one MI355X). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from state_space_model_sscan_amd import binding as bd
    from state_space_model_sscan_amd import inputs as gen

    bd.lib()  # fails loudly if libsscan.so is missing
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)

    log("bench: workload 1 (main)")
    m = bench_mamba1(1, args.steps, args.warmup, torch, bd, gen)
    extra = {}
    if not args.only_main:
        log("bench: workload 3")
        m3 = bench_mamba1(3, max(10, args.steps // 4), 3, torch, bd, gen)
        log("bench: workload 4 (SSD)")
        s4 = bench_ssd(max(10, args.steps // 4), 3, torch, bd, gen)
        log("bench: workload 2 (decode steps)")
        st = bench_step(torch, bd, gen)
        log("bench: conv1d + silu, gated RMS norm")
        conv_e, norm_e = bench_mixer_ops(max(10, args.steps // 4), 3, torch, bd, s4)
        log("bench: Mamba-2 decode steps")
        sst = bench_ssd_step(torch, bd, s4)
        log("bench: hidden attention map")
        att = bench_attention(max(5, args.steps // 10), 2, torch, bd, s4)
        log("bench: SSD with per-token states")
        sts = bench_ssd_states(max(5, args.steps // 10), 2, torch, bd, gen)
        extra = dict(
            mamba1_falcon_width={k: v for k, v in m3.items() if k != "inp"},
            ssd_mamba2_2p7b={k: v for k, v in s4.items() if k not in ("inp", "base")},
            decode_step=st,
            ssd_decode_step=sst,
            conv1d_silu=conv_e,
            gated_rmsnorm=norm_e,
            ssd_attention_map=att,
            ssd_per_token_states=sts,
        )
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(m["inp"])

    inp = m["inp"]
    valu_frac = m["valu_tslots"] / VALU_PEAK_TSLOTS
    tr = recorded_traffic("mamba1_workload1")
    traffic = None if tr is None else tr["hbm_bytes_per_launch"]
    line = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": m["workload"], "batch": inp.batch, "seq_len": inp.seqlen,
                   "channels": inp.channels, "state_dim": inp.state_dim, "ngroups": inp.ngroups,
                   "gate": True, "state": "fp32"},
        "roofline": {"bound": "alu", "achieved": m["valu_tslots"], "peak": VALU_PEAK_TSLOTS,
                     "unit": "T VALU-slots/s", "frac": valu_frac, "traffic": traffic,
                     "kernel": MAIN_KERNEL, "kernel_ms": m["kernel_ms"],
                     "hbm_gbs": m["hbm_gbs"], "hbm_frac": m["hbm_frac"], "algorithmic_bytes": m["bytes"],
                     "updates_per_s": m["updates_per_s"]},
        "cpu_baseline": cpu,
        "secondary": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
