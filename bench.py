"""Benchmark of the selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-counters] [--only-main]

A step is one sscan_mamba1_fwd over the Mamba-130m layer workload (batch 8,
seq 2048, d_inner 1536, state_dim 16, bf16 activations, fp32 state, fused
silu(z) gate). Inputs are resident in HBM when timing starts; three copies of
them rotate so no step finds its inputs in the 256 MiB Infinity Cache. Before
the W warmup steps half a second of VALU work (zeta over a buffer; no step of the
workload) brings the GPU from its idle clock to its loaded one. K steps are then
timed between two device synchronizations, with one pair of HIP events on the
stream the kernels are launched on around them (the kernel time per launch is
their time / K); a second pass of K calls, each between its own events, gives
the median and minimum of single launches. The Falcon-Mamba-7b-width Mamba-1 workload and the Mamba-2 2.7B
SSD workload get blocks of their own with the same roofline and CPU-baseline
fields; beside them the decode steps, the conv1d + silu and gated RMS norm
around the Mamba-2 scan, the hidden attention map and the SSD with per-token
states are reported.

Roofline: every scan is HBM-bound by its arithmetic intensity; `achieved` is the
workload's algorithmic bytes (every input read once, every output written once)
over the kernel time, against the 8 TB/s peak. `traffic` is what the hardware
counters saw: before any GPU work of its own, the bench runs itself under
rocprofv3 as a child (--counter-child) in four counter passes (FETCH_SIZE;
WRITE_SIZE; VALU instruction and busy counters; MFMA counters) and scales the
byte counters by what they read for a plain elementwise kernel that reads and
writes 1 GiB. The SSD block adds the MFMA FLOPs those counters count. The CPU
baseline is the fp64 oracle on bounded samples of the same workloads, timed on
this host's cores (also on one core for the main workload). Prints one JSON line.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import signal
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
VALU_CLOCK_HZ = 2.4e9            # MI355X peak engine clock, published
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, published
F32_MFMA_PEAK_TFLOPS = 157.3     # dense fp32 MFMA, published
MFMA_FLOPS_PER_MOP = 512         # SQ_INSTS_VALU_MFMA_MOPS_* counts units of 512 FLOPs
DEVICE_WARMUP_S = 0.5         # seconds of VALU work before each timed region (device_warmup)
METRIC = "scan tokens/s & % HBM roofline (Mamba-1); SSD tokens/s & % MFMA peak"
MAIN = 1
BLOCKS = (3, 4)                  # the other throughput workloads, with blocks of their own
# Repetitions per workload in the counter child: distinct counts let the parent
# tell the dispatches of each workload apart in the counter records.
COUNTER_REPS = {1: 7, 3: 9, 4: 11}
CALIB_REPS = 13
COUNTER_PASSES = [
    ("read", ["FETCH_SIZE"]),
    ("write", ["WRITE_SIZE"]),
    ("valu", ["SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
              "SQ_WAIT_INST_ANY", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"]),
    ("mfma", ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]),
]
NUM_CU, NUM_XCD = 256, 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- workloads and their byte / FLOP counts
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


def ssd_flops(inp, Q):
    """Contraction FLOPs of the chunked SSD at chunk Q (dense Q x Q blocks): C.B^T per
    (batch, chunk, group), and per (batch, chunk, head) the diagonal block M.X, the chunk
    state X^T.(B*w) and the off-diagonal read C.H^T."""
    b, L, H, P, N, G = inp.batch, inp.seqlen, inp.nheads, inp.head_dim, inp.state_dim, inp.ngroups
    nch = -(-L // Q)
    return b * nch * (G * 2 * Q * Q * N + H * (2 * Q * Q * P + 2 * Q * N * P + 2 * Q * N * P))


def make(gen, wid):
    return gen.make_workload(wid)


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


def scan_call(inp, bd, torch, base):
    """A closure that runs the workload's scan once on a set of its inputs."""
    if hasattr(inp, "channels"):
        b, Dc, N = inp.batch, inp.channels, inp.state_dim
        y = torch.empty_like(base["x"])
        h = torch.empty((b, Dc, N), dtype=torch.float32, device="cuda")
        ws_n = bd.sscan_mamba1_workspace_size(bd.mamba1_desc(base["x"], base["B"], inp.bc_eps))
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

        def fn(s):
            bd.sscan_mamba1_fwd(s["x"], s["dt_raw"], s["dt_bias"], s["A_log"], s["B"], s["C"], s["D"], s["z"],
                                s["state_input"], y=y, state_output=h, workspace=ws, bc_rms_eps=inp.bc_eps)
        return fn
    b, H, P, N = inp.batch, inp.nheads, inp.head_dim, inp.state_dim
    y = torch.empty_like(base["x"])
    h = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    ws_n = bd.sscan_ssd_workspace_size(bd.ssd_desc(base["x"], base["B"], inp.chunk))
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

    def fn(s):
        bd.sscan_ssd_fwd(s["x"], s["dt_raw"], s["dt_bias"], s["A_log"], s["B"], s["C"], s["D"], s["z"],
                         s["state_input"], y=y, state_output=h, workspace=ws, chunk=inp.chunk)
    return fn


def device_warmup(torch, seconds=None):
    """Brings the GPU to its loaded clock before a timed region: Hurwitz zeta over a
    64 MB buffer (a long VALU loop per element, about 0.75 ms per launch, so that a
    kernel trace of the bench stays small) for `seconds`. It is no step of any
    workload. After seconds of host-only work (the CPU baseline, input generation)
    the GPU idles at a low clock: measured cold, the Mamba-130m layer's first tens
    of calls ran 15% slower than after half a second of VALU work (a bf16 GEMM
    warms it less: under MFMA load the clock settles lower)."""
    seconds = DEVICE_WARMUP_S if seconds is None else seconds
    if seconds <= 0:
        return
    x = torch.rand(1 << 24, device="cuda") + 1.5
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        torch.special.zeta(x, 2.0)
        torch.cuda.synchronize()
    del x


def time_calls(fn, sets, steps, warmup, torch):
    """The device warm-up, `warmup` untimed calls, then `steps` timed calls between two
    synchronizations, bracketed by one pair of HIP events on the current stream (the
    one the library launches on), so nothing is queued between the calls. Then, after
    the timed region, the same number of calls with an event pair around each, for
    the spread of single launches. Returns (wall ms per step, event ms statistics:
    `mean` = the timed region's event time / steps, the per-launch GPU time including
    the gaps between launches; `median`, `min`, `per_call_mean` from the second pass)."""
    device_warmup(torch)
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fn(sets[i % len(sets)])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    region = e0.elapsed_time(e1) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        fn(sets[i % len(sets)])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    return wall, dict(mean=float(region), median=float(np.median(ms)), min=float(ms.min()),
                      per_call_mean=float(ms.mean()), n=int(ms.size))


# ---------------------------------------------------------------- hardware counters (rocprofv3 children)
def counter_child():
    """Runs under rocprofv3: each throughput workload COUNTER_REPS times, then a plain
    elementwise kernel of known traffic (reads 1 GiB, writes 1 GiB) CALIB_REPS times."""
    import torch

    from state_space_model_sscan_amd import binding as bd
    from state_space_model_sscan_amd import inputs as gen

    bd.lib()
    for wid, reps in COUNTER_REPS.items():
        inp = make(gen, wid)
        base = upload(inp, torch)
        fn = scan_call(inp, bd, torch, base)
        for _ in range(reps):
            fn(base)
        torch.cuda.synchronize()
        log("counter child: workload %d x %d" % (wid, reps))
        del base, fn
        torch.cuda.empty_cache()
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(CALIB_REPS):
        torch.add(a, 1.0, out=b)
    torch.cuda.synchronize()
    log("counter child: calibration x %d" % CALIB_REPS)


def _read_counters(outdir):
    """{(kernel name, grid): {counter: [values per dispatch]}} from a rocprofv3 csv."""
    files = glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True)
    rec = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"], int(r["Grid_Size"]))
                disp = int(r["Dispatch_Id"])
                rec.setdefault(key, {}).setdefault(r["Counter_Name"], {}).setdefault(disp, 0.0)
                # counters come per die / shader engine in some versions: sum them per dispatch
                rec[key][r["Counter_Name"]][disp] += float(r["Counter_Value"])
    return {k: {c: list(d.values()) for c, d in v.items()} for k, v in rec.items()}


def collect_counters(top=None, timeout_s=240):
    """The four counter passes of the workloads, each in a child process under rocprofv3,
    writing their csv files under `top` (a new temporary directory when None). Must run
    before this process touches the GPU. Returns {pass: records} or an error."""
    prof = shutil.which("rocprofv3")
    if not prof:
        return {"error": "rocprofv3 not found"}
    if top is None:
        import tempfile
        top = tempfile.mkdtemp(prefix="sscan_bench_counters_")
    out = {}
    for name, counters in COUNTER_PASSES:
        d = os.path.join(top, name)
        shutil.rmtree(d, ignore_errors=True)
        os.makedirs(d, exist_ok=True)
        cmd = [prof, "--pmc", *counters, "--output-format", "csv", "-d", d, "-o", "run", "--",
               sys.executable, os.path.abspath(__file__), "--counter-child"]
        log("bench: counter pass %s (%s)" % (name, " ".join(counters)))
        env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
        p = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=open(os.path.join(d, "child.log"), "w"),
                             cwd="/tmp", env=env, start_new_session=True)
        try:
            rc = p.wait(timeout=timeout_s)
        except subprocess.TimeoutExpired:
            os.killpg(p.pid, signal.SIGKILL)
            p.wait()
            return {"error": "counter pass %s timed out" % name}
        rec = _read_counters(d)
        if not rec:  # rocprofv3 may end with a fault after writing whole results; only no data is an error
            return {"error": "counter pass %s wrote no records (rc %d)" % (name, rc)}
        out[name] = rec
    return out


def _by_reps(rec, reps, counter):
    """Mean per dispatch of `counter` over every sscan kernel launched `reps` times,
    summed over those kernels, and the largest of them (name, mean)."""
    total, top = 0.0, (None, -1.0)
    for (kname, grid), cs in rec.items():
        v = cs.get(counter)
        if "sscan::" not in kname or v is None or len(v) != reps:
            continue
        m = float(np.mean(v))
        total += m
        if m > top[1]:
            top = (kname, m)
    return total, top


def _calibration(rec, counter):
    best = None
    for (kname, grid), cs in rec.items():
        v = cs.get(counter)
        if "elementwise" in kname and v is not None and len(v) == CALIB_REPS:
            if best is None or grid > best[0]:
                best = (grid, float(np.mean(v)))
    return None if best is None else best[1]


def counter_summary(cnt, wid, inp):
    """Per workload: HBM bytes per call from FETCH_SIZE / WRITE_SIZE (scaled by the
    calibration kernel's readings), VALU or MFMA figures."""
    if not cnt or "error" in cnt:
        return dict(error=(cnt or {}).get("error", "not collected"))
    reps = COUNTER_REPS[wid]
    rd, (kname, _) = _by_reps(cnt["read"], reps, "FETCH_SIZE")
    wr, _ = _by_reps(cnt["write"], reps, "WRITE_SIZE")
    cf = _calibration(cnt["read"], "FETCH_SIZE")
    cw = _calibration(cnt["write"], "WRITE_SIZE")
    gib_kib = float(1 << 20)  # 1 GiB in KiB
    s = dict(kernel=kname)
    if cf and cw and rd > 0:
        fr, fw = gib_kib / cf, gib_kib / cw
        s.update(read_bytes=rd * 1024 * fr, write_bytes=wr * 1024 * fw,
                 calibration=dict(fetch_size_kib=cf, write_size_kib=cw, fetch_scale=fr, write_scale=fw,
                                  kernel="torch elementwise add, 1 GiB read + 1 GiB written"))
        s["traffic_bytes"] = s["read_bytes"] + s["write_bytes"]
    v = cnt.get("valu", {})
    insts, _ = _by_reps(v, reps, "SQ_INSTS_VALU")
    active, _ = _by_reps(v, reps, "SQ_ACTIVE_INST_VALU")
    trans, _ = _by_reps(v, reps, "SQ_INSTS_VALU_TRANS_F32")
    gui, _ = _by_reps(v, reps, "GRBM_GUI_ACTIVE")
    if insts > 0 and gui > 0:
        units = inp.batch * inp.seqlen * (inp.channels * inp.state_dim if hasattr(inp, "channels")
                                          else inp.nheads * inp.head_dim * inp.state_dim)
        s["valu"] = dict(wave_instructions=insts, transcendental=trans,
                         instructions_per_state_update=insts * 64 / units,
                         busy=active / NUM_CU / (gui / NUM_XCD),
                         note="busy = SQ_ACTIVE_INST_VALU / CUs / GRBM_GUI_ACTIVE per die (rocprof's VALUBusy)")
    m = cnt.get("mfma", {})
    mops, _ = _by_reps(m, reps, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    if mops > 0:
        s["mfma_flops"] = mops * MFMA_FLOPS_PER_MOP
        busy, _ = _by_reps(m, reps, "SQ_VALU_MFMA_BUSY_CYCLES")
        gui, _ = _by_reps(m, reps, "GRBM_GUI_ACTIVE")
        if gui > 0:
            s["mfma_busy"] = busy / (NUM_CU * 4) / (gui / NUM_XCD)
    return s


# ---------------------------------------------------------------- the CPU baseline (the oracle)
def host_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(cpu_model=model, cpu_count=os.cpu_count(), omp_num_threads=os.environ.get("OMP_NUM_THREADS"))


def cpu_baseline(inp, min_seconds, threads=None, sample=None):
    """The fp64 oracle as it stands on `inp` (or a slice of its batch rows), run back to back
    until at least `min_seconds` are timed. Returns tokens/s and state updates/s."""
    import oracle

    oracle.build(force=False)
    full = oracle.threads()
    if threads:
        oracle.set_threads(threads)
    try:
        used = oracle.threads()
        runs, total = 0, 0.0
        while runs < 1 or total < min_seconds:
            t0 = time.perf_counter()
            oracle.run_inputs(inp, want_states=False)
            total += time.perf_counter() - t0
            runs += 1
    finally:
        oracle.set_threads(full)
    per_tok = inp.channels * inp.state_dim if hasattr(inp, "channels") else inp.nheads * inp.head_dim * inp.state_dim
    toks = inp.batch * inp.seqlen * runs
    return dict(value=toks / total, unit="tokens/s", cores=used, kind="oracle",
                updates_per_s=toks * per_tok / total,
                sample="%s, fp64, run %d times back to back, %.1f s in all" % (sample, runs, total))


def batch_rows(inp, rows):
    """The same workload restricted to its first `rows` batch rows (rows are independent)."""
    import copy
    s = copy.copy(inp)
    for k in ("x", "dt_raw", "z", "B", "C", "h0"):
        v = getattr(inp, k)
        if v is not None:
            setattr(s, k, v[:rows])
    s.batch = rows
    return s


# ---------------------------------------------------------------- GPU timing of the workloads
def bench_workload(wid, steps, warmup, torch, bd, gen, inp=None):
    inp = inp or make(gen, wid)
    base = upload(inp, torch)
    sets = [base] + [clone_set(base) for _ in range(2)]
    fn = scan_call(inp, bd, torch, base)
    wall, ev = time_calls(fn, sets, steps, warmup, torch)
    del sets, base
    torch.cuda.empty_cache()
    ssd = not hasattr(inp, "channels")
    by = ssd_bytes(inp) if ssd else mamba1_bytes(inp)
    per_tok = inp.nheads * inp.head_dim * inp.state_dim if ssd else inp.channels * inp.state_dim
    tokens = inp.batch * inp.seqlen
    ksec = ev["mean"] * 1e-3
    d = dict(workload=gen.WORKLOADS[wid]["name"], ms_per_step=wall, kernel_ms=ev, tokens=tokens,
             tokens_per_s=tokens / (wall * 1e-3), updates_per_s=tokens * per_tok / ksec, bytes=by)
    d["roofline"] = dict(bound="hbm", achieved=by / ksec / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=by / ksec / 1e9 / HBM_PEAK_GBS, traffic=None, algorithmic_bytes=by,
                         kernel_ms=ev["mean"])
    if ssd:
        q64, q256 = ssd_flops(inp, 64), ssd_flops(inp, 256)
        d["mfma"] = dict(peak_tflops=BF16_MFMA_PEAK_TFLOPS, counted_flops=None, frac=None,
                         algorithmic_flops_q64=q64, frac_algorithmic_q64=q64 / ksec / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                         algorithmic_flops_q256=q256,
                         frac_algorithmic_q256=q256 / ksec / 1e12 / BF16_MFMA_PEAK_TFLOPS)
    return d, inp


def attach_counters(d, cs):
    d["counters"] = cs
    r = d["roofline"]
    if "traffic_bytes" in cs:
        r["traffic"] = cs["traffic_bytes"]
        r["traffic_read"] = cs["read_bytes"]
        r["traffic_write"] = cs["write_bytes"]
        r["traffic_over_algorithmic"] = cs["traffic_bytes"] / r["algorithmic_bytes"]
        r["counter_kernel"] = cs.get("kernel")
    if "valu" in cs:
        r["valu"] = dict(cs["valu"])
        # VALU issue against its peak: a wave64 VALU instruction occupies a SIMD for 4
        # cycles and a transcendental for 8 (measured), so the counted instructions
        # need (all + transcendental) * 4 SIMD-cycles; the chip has 256 CUs x 4 SIMDs at
        # 2.4 GHz over the kernel's time
        ksec = d["kernel_ms"]["mean"] * 1e-3
        need = (cs["valu"]["wave_instructions"] + cs["valu"]["transcendental"]) * 4
        have = NUM_CU * 4 * VALU_CLOCK_HZ * ksec
        r["valu"]["issue_frac"] = need / have
        r["valu"]["issue_note"] = ("(SQ_INSTS_VALU + SQ_INSTS_VALU_TRANS_F32) x 4 SIMD-cycles over "
                                   "256 CUs x 4 SIMDs x 2.4 GHz x the kernel time")
    if "mfma" in d and "mfma_flops" in cs:
        ksec = d["kernel_ms"]["mean"] * 1e-3
        m = d["mfma"]
        m["counted_flops"] = cs["mfma_flops"]
        m["tflops"] = cs["mfma_flops"] / ksec / 1e12
        m["frac"] = m["tflops"] / BF16_MFMA_PEAK_TFLOPS
        m["busy"] = cs.get("mfma_busy")


# ---------------------------------------------------------------- secondary measurements (the steps next to the scan)
def bench_step(torch, bd, gen, calls=512):
    """Workload 2 as `calls` one-token sscan_step calls, state updated in place: timed
    eagerly (includes the Python/ctypes cost of each call) and as a HIP graph that
    replays the same `calls` launches (the GPU-side cost per step)."""
    inp = make(gen, 2)
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

    device_warmup(torch)
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


def hbm_entry(workload, ms_wall, ev, nbytes, **kw):
    ms = ev["mean"]
    d = dict(workload=workload, ms_per_step=ms_wall, kernel_ms=ev, bytes=nbytes,
             hbm_gbs=nbytes / (ms * 1e-3) / 1e9, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    d.update(kw)
    return d


def bench_mixer_ops(steps, warmup, torch, bd, L=8192, b=4):
    """The steps next to the scan at the Mamba-2 2.7B layer shape (batch 4, 8192 tokens):
    conv1d + silu over xBC (5120 + 2 x 128 = 5376 channels, width 4, with the carried conv
    state in and out), and the gated RMS norm over y, z (80 heads x 64 = 5120 wide). Both
    stream more than the 256 MiB Infinity Cache per call."""
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
    rows, width = b * L, 5120
    y2 = torch.randn((rows, width), generator=g, device="cuda").to(torch.bfloat16)
    z2 = torch.randn((rows, width), generator=g, device="cuda").to(torch.bfloat16)
    wn = torch.rand((width,), generator=g, device="cuda") + 0.5
    nout = torch.empty_like(y2)

    def norm(_):
        bd.sscan_gated_rmsnorm(y2, z2, wn, 1e-5, out=nout)

    wall, ev = time_calls(norm, [None], steps, warmup, torch)
    nbytes = 3 * rows * width * 2 + width * 4
    norm_e = hbm_entry("mamba2-2.7b gated RMS norm, bf16 %d rows x %d" % (rows, width), wall, ev, nbytes,
                       tokens_per_s=rows / (wall * 1e-3))
    return conv_e, norm_e


def bench_ssd_step(torch, bd, gen, nstates=32, calls=64):
    """Mamba-2 2.7B decode: one-token sscan_ssd_step calls at batch 4 (state [4, 80, 64, 128]
    fp32, 10.5 MB, updated in place). The calls cycle over `nstates` separate states, 336 MB
    in all, so that no call finds its state in the 256 MiB Infinity Cache, as in a model whose
    other layers' states pass through between two steps of a layer. Timed as a HIP graph
    that replays `calls` launches."""
    inp = gen.make_workload(4, seqlen=calls)
    base = upload(inp, torch)
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
    device_warmup(torch)
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


def bench_ssd_f32(steps, warmup, torch, bd, gen):
    """sscan_ssd_fwd with fp32 activations at the Mamba-2 2.7B layer shape, one batch row
    (8192 tokens x 80 heads x 64, state 128): the fp32 MFMA chunk kernel, and beside it
    the same call sent to the fp32 token loop (16 lanes per head_dim column) by the
    tuning knob, the path fp32 activations of other shapes take. One batch row has 80
    chains for 256 compute units, so the plan takes two passes (`one_pass`: the same call
    forced to one pass); `full_batch` times the layer's whole batch of 4 (320 chains, one
    pass) on the chunk kernel."""
    inp = gen.make_workload(4, batch=1, act="f32")
    base = upload(inp, torch)
    b, L, H, P, N = inp.batch, inp.seqlen, inp.nheads, inp.head_dim, inp.state_dim
    y = torch.empty_like(base["x"])
    h = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")

    def run(token_loop, one_pass=False):
        prev = bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, 1 if token_loop else 0)
        prev_tp = bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 1 if one_pass else 0)
        try:
            ws_n = bd.sscan_ssd_workspace_size(bd.ssd_desc(base["x"], base["B"], inp.chunk))
            ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")

            def fn(_):
                bd.sscan_ssd_fwd(base["x"], base["dt_raw"], base["dt_bias"], base["A_log"], base["B"], base["C"],
                                 base["D"], base["z"], base["state_input"], y=y, state_output=h, workspace=ws,
                                 chunk=inp.chunk)

            return time_calls(fn, [None], steps, warmup, torch)
        finally:
            bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, prev)
            bd.set_tuning(bd.TUNE_SSD_TWO_PASS, prev_tp)

    wall, ev = run(False)
    owall, oev = run(False, one_pass=True)
    lwall, lev = run(True)
    del base, y, h
    torch.cuda.empty_cache()
    # the whole batch of the layer (4 rows: 320 chains, enough to fill the chip)
    full = gen.make_workload(4, act="f32")
    fb = upload(full, torch)
    fy = torch.empty_like(fb["x"])
    fh = torch.empty((full.batch, H, P, N), dtype=torch.float32, device="cuda")
    fws = torch.empty(max(bd.sscan_ssd_workspace_size(bd.ssd_desc(fb["x"], fb["B"], full.chunk)), 1),
                      dtype=torch.uint8, device="cuda")

    def ffn(_):
        bd.sscan_ssd_fwd(fb["x"], fb["dt_raw"], fb["dt_bias"], fb["A_log"], fb["B"], fb["C"], fb["D"], fb["z"],
                         fb["state_input"], y=fy, state_output=fh, workspace=fws, chunk=full.chunk)

    fwall, fev = time_calls(ffn, [None], max(3, steps // 2), warmup, torch)
    del fb, fy, fh, fws
    torch.cuda.empty_cache()
    fq = ssd_flops(full, 64)
    return hbm_entry("mamba2-2.7b layer, fp32 activations, 1 x 8192 tokens x 80 heads x 64, state 128 "
                     "(fp32 MFMA chunk kernel)", wall, ev, ssd_bytes(inp), tokens_per_s=b * L / (wall * 1e-3),
                     updates_per_s=b * L * H * P * N / (ev["mean"] * 1e-3),
                     mfma_flops_q64=ssd_flops(inp, 64),
                     mfma_frac_fp32_q64=ssd_flops(inp, 64) / (ev["mean"] * 1e-3) / 1e12 / F32_MFMA_PEAK_TFLOPS,
                     one_pass=dict(ms_per_step=owall, kernel_ms=oev, tokens_per_s=b * L / (owall * 1e-3)),
                     token_loop=dict(ms_per_step=lwall, kernel_ms=lev, tokens_per_s=b * L / (lwall * 1e-3)),
                     full_batch=dict(workload="4 x 8192 tokens x 80 heads x 64, state 128, fp32", ms_per_step=fwall,
                                     kernel_ms=fev, tokens_per_s=full.batch * L / (fwall * 1e-3),
                                     hbm_frac=ssd_bytes(full) / (fev["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                     mfma_frac_fp32_q64=fq / (fev["mean"] * 1e-3) / 1e12 / F32_MFMA_PEAK_TFLOPS))


def bench_ssd_one_row(steps, warmup, torch, bd, gen):
    """The Mamba-2 2.7B layer's SSD for one batch row (bf16, 8192 tokens x 80 heads): 80
    chains for 256 compute units, so the plan takes two passes; `one_pass` is the same
    call forced to one pass (segments handing their states on in turn)."""
    inp = gen.make_workload(4, batch=1)
    d, _ = bench_workload(4, steps, warmup, torch, bd, gen, inp)
    d["workload"] = "mamba2-2.7b layer, one batch row, bf16 (1 x 8192 tokens x 80 heads x 64, state 128)"
    prev = bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 1)
    try:
        o, _ = bench_workload(4, steps, warmup, torch, bd, gen, inp)
    finally:
        bd.set_tuning(bd.TUNE_SSD_TWO_PASS, prev)
    d["one_pass"] = dict(ms_per_step=o["ms_per_step"], kernel_ms=o["kernel_ms"], tokens_per_s=o["tokens_per_s"])
    return d


def bench_ssd_shape(steps, warmup, torch, bd, gen, label, **overrides):
    """The Mamba-2 2.7B layer's SSD (bf16, 4 x 8192 tokens) at another head or state
    shape on the bf16 chunk kernel: 40 heads of 128 columns (the same channels; each head
    runs as two 64-column heads sharing its step and decay), or state_dim 64 (B, C and
    the states zero-padded to 128 in the workspace, so the kernel does the work of 128;
    the padding and un-padding kernels are in the call's time)."""
    inp = gen.make_workload(4, **overrides)
    d, _ = bench_workload(4, steps, warmup, torch, bd, gen, inp)
    d["workload"] = label
    return d


def bench_ssd_split(steps, warmup, torch, bd, gen):
    """The Mamba-2 2.7B layer's SSD (bf16, 4 x 8192 tokens) in the precise form of the
    bf16 chunk path (SSCAN_TUNE_SSD_SPLIT_STATE: the state as C reads it and w x as two
    bf16 parts each, twice the MFMAs of those two products)."""
    prev = bd.set_tuning(bd.TUNE_SSD_SPLIT_STATE, 1)
    try:
        d, _ = bench_workload(4, steps, warmup, torch, bd, gen, gen.make_workload(4))
    finally:
        bd.set_tuning(bd.TUNE_SSD_SPLIT_STATE, prev)
    d["workload"] = "mamba2-2.7b layer, bf16, precise form (state and w x as two bf16 parts)"
    return d


def bench_attention(steps, warmup, torch, bd, gen, L=2048):
    """The hidden attention map of the first L tokens of one batch row of the Mamba-2 2.7B
    workload's distributions (80 heads, one group, state 128): alpha [1, L, L, 80] fp32,
    1.34 GB written per call."""
    inp = gen.make_workload(4, batch=1, seqlen=L)
    dt = upload(inp, torch)
    H = inp.nheads
    alpha = torch.empty((1, L, L, H), dtype=torch.float32, device="cuda")

    def fn(_):
        bd.sscan_ssd_attention(dt["dt_raw"], dt["dt_bias"], dt["A_log"], dt["B"], dt["C"], alpha=alpha)

    wall, ev = time_calls(fn, [None], steps, warmup, torch)
    nbytes = L * L * H * 4 + L * H * 2 + 2 * L * inp.ngroups * inp.state_dim * 2 + 2 * H * 4
    return hbm_entry("mamba2-2.7b hidden attention map, 1 x %d tokens x %d heads, fp32 out" % (L, H), wall, ev,
                     nbytes)


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-counters", action="store_true", help="skip the rocprofv3 counter passes")
    ap.add_argument("--only-main", action="store_true", help="time only the main workload")
    ap.add_argument("--counter-dir", default=None, help="where the counter passes write their csv files "
                    "(default: a new temporary directory)")
    ap.add_argument("--counter-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (every box has one MI355X). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.counter_child:
        counter_child()
        return

    from state_space_model_sscan_amd import binding as bd
    from state_space_model_sscan_amd import inputs as gen

    bd.lib()  # fails loudly if libsscan.so is missing
    # Child processes first (the counter passes), before this process touches the GPU.
    cnt = None
    if not args.no_counters and not args.only_main:
        cnt = collect_counters(args.counter_dir)
        if "error" in cnt:
            log("bench: counters unavailable: %s" % cnt["error"])

    log("bench: inputs")
    inputs = {MAIN: make(gen, MAIN)}
    if not args.only_main:
        for w in BLOCKS:
            inputs[w] = make(gen, w)

    cpu = {}
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        m = inputs[MAIN]
        cpu[MAIN] = cpu_baseline(m, 10.0, sample="the whole workload (%d x %d tokens x %d channels x %d states)"
                                 % (m.batch, m.seqlen, m.channels, m.state_dim))
        one = batch_rows(m, 1)
        cpu[MAIN]["single_thread"] = cpu_baseline(one, 3.0, threads=1,
                                                  sample="batch row 0 of the workload (1 x %d tokens x %d channels)"
                                                  % (m.seqlen, m.channels))
        if not args.only_main:
            w3 = inputs[3]
            cpu[3] = cpu_baseline(w3, 5.0, sample="the whole workload (%d x %d tokens x %d channels x %d states)"
                                  % (w3.batch, w3.seqlen, w3.channels, w3.state_dim))
            w4 = batch_rows(inputs[4], 1)
            cpu[4] = cpu_baseline(w4, 3.0, sample="batch row 0 of the workload (1 x %d tokens x %d heads x %d x %d "
                                  "states)" % (w4.seqlen, w4.nheads, w4.head_dim, w4.state_dim))

    import torch

    torch.cuda.set_device(0)
    log("bench: workload %d (main)" % MAIN)
    main_d, _ = bench_workload(MAIN, args.steps, args.warmup, torch, bd, gen, inputs[MAIN])
    if cnt:
        attach_counters(main_d, counter_summary(cnt, MAIN, inputs[MAIN]))
    blocks, extra = {}, {}
    if not args.only_main:
        for w in BLOCKS:
            log("bench: workload %d" % w)
            d, _ = bench_workload(w, max(10, args.steps // 4), 3, torch, bd, gen, inputs[w])
            if cnt:
                attach_counters(d, counter_summary(cnt, w, inputs[w]))
            d["cpu_baseline"] = cpu.get(w)
            blocks[d["workload"]] = d
        del inputs
        log("bench: decode steps")
        extra["decode_step"] = bench_step(torch, bd, gen)
        log("bench: conv1d + silu, gated RMS norm")
        extra["conv1d_silu"], extra["gated_rmsnorm"] = bench_mixer_ops(max(10, args.steps // 4), 3, torch, bd)
        log("bench: Mamba-2 decode steps")
        extra["ssd_decode_step"] = bench_ssd_step(torch, bd, gen)
        log("bench: hidden attention map")
        extra["ssd_attention_map"] = bench_attention(max(5, args.steps // 10), 2, torch, bd, gen)
        log("bench: SSD with per-token states")
        extra["ssd_per_token_states"] = bench_ssd_states(max(5, args.steps // 10), 2, torch, bd, gen)
        log("bench: SSD with fp32 activations")
        extra["ssd_fp32"] = bench_ssd_f32(max(3, args.steps // 10), 1, torch, bd, gen)
        log("bench: SSD, one batch row")
        extra["ssd_one_row"] = bench_ssd_one_row(max(5, args.steps // 4), 3, torch, bd, gen)
        log("bench: SSD with head_dim 128, with state_dim 64")
        extra["ssd_head_dim_128"] = bench_ssd_shape(
            max(5, args.steps // 4), 3, torch, bd, gen,
            "mamba2-2.7b layer as 40 heads x 128 columns, state 128, bf16 (4 x 8192 tokens)", nheads=40, head_dim=128)
        extra["ssd_state_dim_64"] = bench_ssd_shape(
            max(5, args.steps // 4), 3, torch, bd, gen,
            "mamba2-2.7b layer with state_dim 64, bf16 (4 x 8192 tokens x 80 heads x 64)", state_dim=64)
        log("bench: SSD, precise form")
        extra["ssd_split_state"] = bench_ssd_split(max(5, args.steps // 4), 3, torch, bd, gen)

    cfg = gen.WORKLOADS[MAIN]
    roof = dict(main_d["roofline"])
    roof["kernel_ms_median"] = main_d["kernel_ms"]["median"]
    roof["kernel_ms_min"] = main_d["kernel_ms"]["min"]
    roof["updates_per_s"] = main_d["updates_per_s"]
    line = {
        "metric": METRIC,
        "value": main_d["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_d["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": cfg["batch"], "seq_len": cfg["seqlen"],
                   "channels": cfg["channels"], "state_dim": cfg["state_dim"], "ngroups": 1,
                   "gate": True, "state": "fp32"},
        "roofline": roof,
        "cpu_baseline": cpu.get(MAIN),
        "kernel_ms": main_d["kernel_ms"],
        "device_warmup_s": DEVICE_WARMUP_S,
        "counters": main_d.get("counters"),
        "host": host_info(),
        "workloads": blocks,
        "secondary": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
