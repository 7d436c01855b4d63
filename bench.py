"""Attention fwd+bwd throughput on one MI355X, against the bf16 MFMA peak.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]

A step is one forward (fa_fwd) plus one backward (fa_bwd) over the
workload's synthetic inputs, already resident in HBM.  Work is counted on
allowed (query, key) pairs only: 4*D flop per pair forward, 10*D backward
(the five contractions QK^T, PV, dO V^T, P^T dO, dS K / dS^T Q), 14*D in all.

Prints one JSON line: the metric, the per-step time, fwd / bwd / fwd+bwd
TFLOP/s and their fraction of the 2516.6 TFLOP/s dense bf16 peak, the time of
each kernel, the roofline of the dominant kernel (the dK/dV stage), the peak
device memory, and the fp64 oracle timed on a bounded sample of the same
workload on the host CPU, and (``platform_gemm``) a dense bf16 GEMM through
the vendor BLAS timed on the same box after the steps: the practical rate of
the matrix cores there, which the kernels' fractions can be read against.
The timed step is fa_fwd then fa_bwd, as a caller
runs them (fa_bwd launches Delta, then dK/dV and dQ as one kernel where the
shapes allow); the per-kernel times come from further steps, outside the
timed ones, that launch the backward's three stages one by one
(fa_bwd_stage) with HIP events between them on the launch stream.

Algorithmic work per allowed pair, by kernel: forward 4*D (S = QK^T, PV);
dK/dV 8*D (S, dP = dO V^T, dV += P^T dO, dK += dS^T Q); dQ 2*D (dQ += dS K;
its recomputation of S and dP is overhead and is not counted); Delta reads
O and dO (4*D bytes per query row in bf16) and does no contraction.

The dK/dV stage is two launches: dkdv_split_kernel (the products; each key
block's query steps split between two workgroups that write float32 partial
sums) and dkdv_reduce_kernel (adds the two halves, about 1 % of the stage's
time); the roofline times them together, as one unit of work.  Its
``traffic`` (HBM bytes per stage) comes from a committed rocprofv3 counter
summary (FETCH_SIZE, WRITE_SIZE of both kernels) whose recorded source hash
must match the current kernel sources, else it is null.

    python bench.py --copy-calibration

runs one 256 MiB device-to-device copy: its FETCH_SIZE/WRITE_SIZE readings
give the factor that turns those counters into bytes.

    python bench.py --sweep [--steps K] [--warmup W]

times every named workload in turn (the tiny fp32 cases, the batch-8 grid,
16K/32K long GQA, the TTT step-2 call, DiT self- and cross-attention) and
prints one JSON line per workload: fwd / bwd / step times, TFLOP/s, the
fraction of the dense peak of the arithmetic type, the attainable rate
min(peak, AI x 8 TB/s) from the algorithmic bytes, and the peak device memory
of one fwd+bwd.  No oracle timing.

    python bench.py --loss [--workload lsm_loss_B1_T16384_V32000] [--loss-all]

times the soft-target log-softmax loss (fa_lsm_loss_fwd + fa_lsm_loss_bwd,
the EAGLE3 loss after attention) on the SpecForge page's (B, T, V)
configurations: one JSON line per configuration with the forward, backward
and step times and their HBM throughput over the algorithmic bytes (forward:
logits and targets read once, 8 bytes per element; backward: both read and
the gradient written over the logits, 12 bytes per element) against the
8 TB/s peak, the peak device memory above the inputs, and (first
configuration only) the fp64 oracle timed on a sample of rows.  The logits
are restored from a pristine copy before each step, outside the timed
events.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0


def pair_count(w):
    """Allowed (query, key) pairs of one (batch, head), per batch entry."""
    out = []
    i = np.arange(w.Sq, dtype=np.int64)
    for b in range(w.B):
        cap = w.Sq if w.kind == W.TTT else w.Skv
        kvv = cap if w.kv_valid is None else min(max(w.kv_valid[b], 0), cap)
        if w.kind == W.FULL:
            out.append(w.Sq * kvv)
            continue
        if w.kind == W.WINDOW:
            left, right = w.window
            lo = np.clip(i - w.shift - left, 0, kvv)
            hi = np.clip(i - w.shift + right + 1, 0, kvv)
            out.append(int(np.maximum(hi - lo, 0).sum()))
            continue
        causal = int(np.clip(i - w.shift + 1, 0, kvv).sum())
        if w.kind == W.CAUSAL:
            out.append(causal)
        else:
            steps = w.Skv // w.Sq
            out.append(causal + (steps - 1) * min(w.Sq, kvv))
    return out


def frozen_pair_count(w):
    """Allowed pairs (per head, summed over batch) whose key is frozen: their
    dK/dV products are not computed (the prefix workloads)."""
    if not getattr(w, "frozen", 0):
        return 0
    return sum(pair_count(w.with_(Skv=min(w.Skv, w.frozen), kv_valid=None if w.kv_valid is None else
                                  tuple(min(x, w.frozen) for x in w.kv_valid))))


def flops(w):
    pairs = sum(pair_count(w)) * w.Hq
    fz = frozen_pair_count(w) * w.Hq
    return 4 * w.D * pairs, 10 * w.D * pairs - 4 * w.D * fz


def algorithmic_bytes(w):
    """HBM bytes the forward and the backward must move at least: the forward
    reads Q, K, V and writes O and LSE; the backward reads Q, K, V, O, dO and
    LSE, writes dQ, dK, dV, and writes and reads Delta."""
    e = 2 if w.dtype == "bf16" else 4
    qsz, kvsz, rows = w.B * w.Hq * w.Sq * w.D, w.B * w.Hkv * w.Skv * w.D, w.B * w.Hq * w.Sq
    fwd = e * (2 * qsz + 2 * kvsz) + 4 * rows
    bwd = e * (4 * qsz + 4 * kvsz) + 4 * rows + 8 * rows
    return fwd, bwd


def kernel_flops(w):
    """Algorithmic flops of one launch of each kernel."""
    pairs = sum(pair_count(w)) * w.Hq
    fz = frozen_pair_count(w) * w.Hq
    return {"fwd": 4 * w.D * pairs, "dkdv": 8 * w.D * (pairs - fz), "dq": 2 * w.D * pairs}


# Sources compiled into the loss kernels (the same rule for their summary).
LOSS_SOURCES = ("flash_attention_fa_amd/csrc/fa_loss.hip", "flash_attention_fa_amd/csrc/fa_internal.h",
                "flash_attention_fa_amd/build.py")
# Sources compiled into the dK/dV kernel: a counter summary taken on other
# sources no longer describes it.
DKDV_SOURCES = ("flash_attention_fa_amd/csrc/fa_bwd.hip", "flash_attention_fa_amd/csrc/fa_device.h",
                "flash_attention_fa_amd/csrc/fa_internal.h", "flash_attention_fa_amd/build.py")


def sources_sha256(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload, sources, prefix="traffic"):
    """HBM bytes per launch from profiles/<prefix>_<kernel>_<workload>.md, or
    None when there is no summary or it was taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_{kernel}_{workload}.md" if kernel else f"{prefix}_{workload}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ")):
            key, _, val = line.partition(":")
            kv[key.strip()] = val.strip()
    if kv.get("sources_sha256") != sources_sha256(sources):
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """One 256 MiB copy for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 256 << 20
    x = torch.ones(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n}), flush=True)
    return 0


def gemm_reference(dev, n=8192, reps=60, rounds=5):
    """A dense n^3 bf16 GEMM through the vendor BLAS (torch.matmul, hipBLASLt on
    ROCm) on this machine: the practical dense-MFMA rate the attention kernels'
    fraction of the peak can be read against.  Context only; no part of the
    attention path uses it."""
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev, generator=g)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev, generator=g)
    for _ in range(5):
        c = a @ b
    torch.cuda.synchronize()
    times = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    ms = float(np.median(times))
    del a, b, c
    return ms, 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def find_workload(name):
    for w in W.all_workloads():
        if w.name == name:
            return w
    raise SystemExit(f"unknown workload {name}; known: {[w.name for w in W.all_workloads()]}")


def cpu_baseline(w, q, k, v, do, nheads):
    """The fp64 oracle, forward and backward, on batch 0 and query heads
    [0, nheads) of the workload (every row), timed on the host; returns the
    JSON object."""
    from threadpoolctl import threadpool_info
    from oracle import attention_ref
    nheads = max(1, min(nheads, w.Hq))
    kvv = None if w.kv_valid is None else list(w.kv_valid)
    args = [x[:1].double().numpy() for x in (q, k, v, do)]
    t0 = time.perf_counter()
    attention_ref(*args, w.kind, w.shift, None if kvv is None else kvv[:1], w.scale,
                  heads=list(range(nheads)), window=w.window)
    sec = time.perf_counter() - t0
    pairs = pair_count(w)[0] * nheads
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": 14 * w.D * pairs / sec / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle, fwd+bwd of batch 0, query heads [0, {nheads}), all "
                      f"{w.Sq} rows, of {w.name} ({pairs} allowed pairs, {sec:.2f} s, "
                      f"host nproc {os.cpu_count()})"}


def dkdv_label(w):
    if w.dtype == "bf16":
        return "dK/dV stage (fa_bwd_stage FA_BWD_DKDV: dkdv_split_kernel + dkdv_reduce_kernel)"
    return "dK/dV stage (fa_bwd_stage FA_BWD_DKDV: one kernel)"


class ClockSampler:
    """Samples the GPU's current shader clock (MHz) from the driver's DPM
    table in sysfs (the level marked '*' in pp_dpm_sclk) every few
    milliseconds on a host thread while the timed steps run.  Where no such
    file is readable the samples stay empty and the clock is reported as
    unknown (never guessed)."""

    def __init__(self, period_s=0.005):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = {}
        self.period = period_s
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        v = line.split(":", 1)[1].strip().rstrip("*").strip().lower()
                        return float(v.replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for p in self.paths:
                v = self._read(p)
                if v is not None:
                    self.samples.setdefault(p, []).append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self):
        """The busiest card's samples (the one under load reads the highest
        median), or None when nothing could be read."""
        if not self.samples:
            return None
        path, vals = max(self.samples.items(), key=lambda kv: float(np.median(kv[1])))
        return {"sclk_mhz_median": float(np.median(vals)), "sclk_mhz_min": float(np.min(vals)),
                "sclk_mhz_max": float(np.max(vals)), "samples": len(vals),
                "source": path + " (DPM level marked '*', sampled during the timed steps)"}


NRUNS = 3


def run_sizes(steps, nruns=NRUNS):
    """The timed steps split into nruns runs (sizes differ by at most one)."""
    nruns = max(1, min(nruns, steps))
    return [steps // nruns + (1 if i < steps % nruns else 0) for i in range(nruns)]


def measure(fa, w, dev, steps, warmup, inputs):
    """Times `steps` fwd+bwd steps of workload w after `warmup` untimed ones,
    with HIP events on the launch stream around the forward and after each
    backward stage.  The timed steps run as three runs separated by a device
    synchronisation (each step itself interleaves the forward and backward
    arms); the clock is sampled throughout."""
    qg, kg, vg, dog = (x.to(dev) for x in inputs)
    kvv = W.kv_valid_tensor(w, dev)
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    ws = torch.empty(max(1, fa.fa_bwd_workspace_bytes(qg, kg, mask_kind=w.kind)), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(1, fa.fa_fwd_workspace_bytes(qg, kg)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    kw = dict(mask_kind=w.kind, causal_shift=w.shift, kv_valid=kvv, scale=w.scale, window=w.window,
              frozen_keys=w.frozen, stream=stream)

    def fwd():
        fa.fa_fwd(qg, kg, vg, out=o, lse=lse, workspace=fws, **kw)

    def bwd():
        # the whole backward, as a caller runs it (fa_bwd: Delta, then dK/dV and dQ)
        fa.fa_bwd(qg, kg, vg, o, lse, dog, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

    def bwd_stages(marks):
        # fa_bwd's three stages launched one by one, an event after each
        for i, stage in enumerate((fa.FA_BWD_DELTA, fa.FA_BWD_DKDV, fa.FA_BWD_DQ)):
            fa.fa_bwd_stage(stage, qg, kg, vg, o, lse, dog, dq, dk, dv, ws, **kw)
            marks[i].record(stream)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    # peak over outputs, workspaces and one fwd+bwd, above the resident inputs
    peak_mem = torch.cuda.max_memory_allocated(dev) - mem0

    # events: step start, fwd end, bwd end (= step end)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    sizes = run_sizes(steps)
    runs = []
    wall = 0.0
    s = 0
    with ClockSampler() as clock:
        for n in sizes:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            first = s
            for _ in range(n):
                ev[s][0].record(stream)
                fwd()
                ev[s][1].record(stream)
                bwd()
                ev[s][2].record(stream)
                s += 1
            torch.cuda.synchronize()
            wall += time.perf_counter() - t0
            runs.append((first, s))
    span = lambda e, i, j: [x[i].elapsed_time(x[j]) for x in e]
    run_ms = [ev[a][0].elapsed_time(ev[b - 1][2]) / (b - a) for a, b in runs]
    run_fwd = [float(np.median([ev[k][0].elapsed_time(ev[k][1]) for k in range(a, b)])) for a, b in runs]
    run_bwd = [float(np.median([ev[k][1].elapsed_time(ev[k][2]) for k in range(a, b)])) for a, b in runs]
    # per-stage times (outside the timed steps): each backward stage launched
    # alone, after a forward, an event after each
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for x in sev:
        fwd()
        x[0].record(stream)
        bwd_stages(x[1:])
    torch.cuda.synchronize()
    # inputs + outputs + workspace resident during the step
    resident = sum(t.numel() * t.element_size() for t in (qg, kg, vg, dog, o, lse, dq, dk, dv, ws, fws))
    return {"fwd_ms": span(ev, 0, 1), "bwd_ms": span(ev, 1, 2),
            "stage_ms": {"delta": span(sev, 0, 1), "dkdv": span(sev, 1, 2), "dq": span(sev, 2, 3)},
            "ms_step": sum(r * n for r, n in zip(run_ms, sizes)) / steps,
            "runs": {"steps": sizes, "ms_per_step": run_ms, "fwd_ms_median": run_fwd, "bwd_ms_median": run_bwd},
            "clock": clock.summary(),
            "peak_mem": int(peak_mem), "resident": int(resident), "mem0": int(mem0), "wall": wall}


def sweep(fa, dev, steps, warmup):
    """One JSON line per named workload (see the module docstring)."""
    for w in W.all_workloads():
        print(json.dumps({"sweep_case": w.name}), flush=True)
        r = measure(fa, w, dev, steps, warmup, W.make_inputs(w, seed=0))
        f_fwd, f_bwd = flops(w)
        b_fwd, b_bwd = algorithmic_bytes(w)
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        fwd_med, bwd_med = float(np.median(r["fwd_ms"])), float(np.median(r["bwd_ms"]))
        tf = lambda f, ms: f / (ms * 1e-3) / 1e12
        att = lambda f, b: min(peak, f / b * PEAK_HBM_GBS / 1e3)
        row = {"workload": w.name, "dtype": w.dtype,
               "config": {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Skv": w.Skv, "D": w.D,
                          "mask": W.KIND_NAMES[w.kind], "kv_valid": w.kv_valid},
               "peak_tflops": peak}
        for name, f, b, ms in (("fwd", f_fwd, b_fwd, fwd_med), ("bwd", f_bwd, b_bwd, bwd_med),
                               ("step", f_fwd + f_bwd, b_fwd + b_bwd, r["ms_step"])):
            row[name] = {"ms": round(ms, 4), "tflops": round(tf(f, ms), 2),
                         "pct_of_peak": round(100 * tf(f, ms) / peak, 2),
                         "ai_flop_per_byte": round(f / b, 1),
                         "attainable_tflops": round(att(f, b), 1),
                         "pct_of_attainable": round(100 * tf(f, ms) / att(f, b), 2)}
        row["stages_ms_mean"] = {n: round(float(np.mean(v)), 4) for n, v in r["stage_ms"].items()}
        row["peak_mem_bytes"] = r["peak_mem"]
        print(json.dumps(row), flush=True)
        torch.cuda.empty_cache()
    return 0


def loss_bench(fa, w, dev, steps, warmup, cpu):
    """One JSON line for the log-softmax loss workload w (see the module
    docstring)."""
    x0, t, mask = W.make_loss_inputs(w, seed=0, device=dev)
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    x = torch.empty_like(x0)
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(marks=None):
        x.copy_(x0)
        if marks:
            marks[0].record(stream)
        loss, row, m, d, tsum = fa.lsm_loss_fwd(x, t, mask, stream=stream)
        if marks:
            marks[1].record(stream)
        fa.lsm_loss_bwd(x, t, mask, m, d, tsum, one, stream=stream)
        if marks:
            marks[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev) - base
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for s_ in range(steps):
        step(ev[s_])
    torch.cuda.synchronize()
    f_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    nv = w.N * w.V
    fb, bb = 8 * nv + 5 * 4 * w.N + 4, 12 * nv + 5 * 4 * w.N
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    st_gbs = gbs(fb + bb, f_ms + b_ms)
    out = {"metric": "soft-target log-softmax loss fwd+bwd HBM GB/s at 1 MI355X",
           "value": round(st_gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
           "ms_per_step": round(f_ms + b_ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded 4*N(0,1) logits, u**8-normalised soft targets, prompt rows masked)",
           "config": {"workload": w.name, "B": w.B, "T": w.T, "V": w.V},
           "fwd": {"ms_median": round(f_ms, 4), "gbs": round(gbs(fb, f_ms), 1)},
           "bwd": {"ms_median": round(b_ms, 4), "gbs": round(gbs(bb, b_ms), 1)},
           "roofline": {"kernel": "lsm_loss_fwd_kernel + lsm_loss_bwd_kernel (+ the mean)", "bound": "hbm",
                        "achieved": round(st_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(st_gbs / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic(None, w.name, LOSS_SOURCES, prefix="kernels"),
                        "traffic_unit": "HBM bytes per step (FETCH_SIZE x2 + WRITE_SIZE x1, copy-calibrated, "
                                        "forward and backward kernels)"},
           "memory": {"peak_above_inputs_bytes": int(peak), "inputs_bytes": int(mem0),
                      "explicit_chain_intermediates_bytes": 4 * nv * 4}}
    if cpu:
        from threadpoolctl import threadpool_info
        from oracle import logsoftmax_loss_forward, logsoftmax_loss_backward
        rows = min(w.N, 256)
        X = x0[:rows].double().cpu().numpy()
        T = t[:rows].double().cpu().numpy()
        M = mask[:rows].double().cpu().numpy()
        t0 = time.perf_counter()
        logsoftmax_loss_forward(X, T, M)
        logsoftmax_loss_backward(X, T, M)
        sec = time.perf_counter() - t0
        threads = max([q.get("num_threads", 1) for q in threadpool_info()] or [1])
        out["cpu_baseline"] = {"value": round((fb + bb) * rows / w.N / sec / 1e9, 3), "unit": "GB/s",
                               "cores": int(threads), "kind": "oracle",
                               "sample": f"fp64 numpy oracle, fwd+bwd of the first {rows} rows of {w.name} "
                                         f"({sec:.2f} s, host nproc {os.cpu_count()})"}
    print(json.dumps(out), flush=True)
    del x, x0, t, mask
    torch.cuda.empty_cache()


def runs_summary(r, f_fwd, f_bwd, tf):
    """The three runs of the timed steps: per-run step, forward and backward
    times, and their median and spread (max - min over the median, %)."""
    rr = r["runs"]
    out = {"steps": rr["steps"], "ms_per_step": [round(x, 4) for x in rr["ms_per_step"]],
           "fwd_ms_median": [round(x, 4) for x in rr["fwd_ms_median"]],
           "bwd_ms_median": [round(x, 4) for x in rr["bwd_ms_median"]]}
    for key in ("ms_per_step", "fwd_ms_median", "bwd_ms_median"):
        v = rr[key]
        med = float(np.median(v))
        out[key.replace("_median", "") + "_median_of_runs"] = round(med, 4)
        out[key.replace("_median", "") + "_spread_pct"] = round(100 * (max(v) - min(v)) / med, 2)
    out["fwd_pct_of_peak_median_of_runs"] = round(
        100 * tf(f_fwd, float(np.median(rr["fwd_ms_median"]))) / PEAK_BF16_TFLOPS, 2)
    out["step_pct_of_peak_median_of_runs"] = round(
        100 * tf(f_fwd + f_bwd, float(np.median(rr["ms_per_step"]))) / PEAK_BF16_TFLOPS, 2)
    return out


PEAK_SCLK_MHZ = 2400.0   # the clock the published dense peak is quoted at


def clock_summary(clock, value):
    """The sampled clock and the fraction of the dense peak scaled to it."""
    if clock is None:
        return {"sclk_mhz_median": None, "source": "no readable pp_dpm_sclk on this host",
                "pct_of_peak_clock_adjusted": None}
    adj = PEAK_BF16_TFLOPS * clock["sclk_mhz_median"] / PEAK_SCLK_MHZ
    return dict(clock, peak_tflops_at_sclk=round(adj, 1),
                pct_of_peak_clock_adjusted=round(100 * value / adj, 2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=W.HEADLINE.name)
    ap.add_argument("--cpu-heads", type=int, default=3,
                    help="query heads of batch 0 the oracle baseline computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the vendor-BLAS bf16 GEMM timed for context after the steps")
    ap.add_argument("--sweep", action="store_true",
                    help="time every named workload, one JSON line each, and exit")
    ap.add_argument("--loss", action="store_true",
                    help="time the soft-target log-softmax loss instead of attention")
    ap.add_argument("--loss-all", action="store_true",
                    help="with --loss: every configuration of the page's loss table")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB device copy (counter calibration) and exit")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(one process drives one GPU; the library does not shard across GPUs)", file=sys.stderr)
        return 2

    if a.copy_calibration:
        return copy_calibration()
    import flash_attention_fa_amd as fa
    dev = torch.device("cuda", int(os.environ.get("LOCAL_RANK", 0)))
    torch.cuda.set_device(dev)
    if a.sweep:
        return sweep(fa, dev, a.steps, a.warmup)
    if a.loss:
        ws = W.loss_workloads() if a.loss_all else \
            [x for x in W.loss_workloads() if x.name == a.workload] or [W.LOSS_HEADLINE]
        for i, lw in enumerate(ws):
            loss_bench(fa, lw, dev, a.steps, a.warmup, cpu=(i == 0 and not a.no_cpu_baseline))
        return 0
    w = find_workload(a.workload)
    q, k, v, do = W.make_inputs(w, seed=0)
    r = measure(fa, w, dev, a.steps, a.warmup, (q, k, v, do))
    fwd_ms, bwd_ms, stage_ms, ms_step = r["fwd_ms"], r["bwd_ms"], r["stage_ms"], r["ms_step"]
    f_fwd, f_bwd = flops(w)
    fwd_med, bwd_med = float(np.median(fwd_ms)), float(np.median(bwd_ms))
    fwd_avg = float(np.mean(fwd_ms))
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    value = tf(f_fwd + f_bwd, ms_step)
    peak_mem, resident, mem0, wall = r["peak_mem"], r["resident"], r["mem0"], r["wall"]

    kf = kernel_flops(w)
    k_avg = {"fwd": fwd_avg, **{n: float(np.mean(v)) for n, v in stage_ms.items()}}
    kernels = {n: {"ms_mean": round(ms, 4)} for n, ms in k_avg.items()}
    for n, f in kf.items():
        kernels[n]["algorithmic_tflops"] = round(tf(f, k_avg[n]), 2)
        kernels[n]["pct_of_peak"] = round(100 * tf(f, k_avg[n]) / PEAK_BF16_TFLOPS, 2)
    # Delta is HBM-bound: reads O and dO, writes one float per row
    delta_bytes = 2 * w.B * w.Hq * w.Sq * w.D * (2 if w.dtype == "bf16" else 4) + 4 * w.B * w.Hq * w.Sq
    kernels["delta"]["gbs"] = round(delta_bytes / (k_avg["delta"] * 1e-3) / 1e9, 1)
    dkdv_tf = tf(kf["dkdv"], k_avg["dkdv"])
    traffic = measured_traffic("dkdv", w.name, DKDV_SOURCES)
    out = {
        "metric": "attention fwd+bwd TFLOP/s and % of bf16 MFMA peak at 1 MI355X (causal S=16K)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) Q, K, V, dO; no dataset)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Skv": w.Skv, "D": w.D, "mask": W.KIND_NAMES[w.kind],
                   "kv_valid": w.kv_valid, "causal_shift": w.shift},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms_median": round(fwd_med, 4), "tflops": round(tf(f_fwd, fwd_med), 2),
                "pct_of_peak": round(100 * tf(f_fwd, fwd_med) / PEAK_BF16_TFLOPS, 2)},
        "bwd": {"ms_median": round(bwd_med, 4), "tflops": round(tf(f_bwd, bwd_med), 2),
                "pct_of_peak": round(100 * tf(f_bwd, bwd_med) / PEAK_BF16_TFLOPS, 2)},
        "gflop_per_step": round((f_fwd + f_bwd) / 1e9, 3),
        "kernels": kernels,
        "kernel_timing": "fwd: the timed steps; delta, dkdv, dq: each backward stage launched alone "
                         "(fa_bwd_stage), in steps after the timed ones",
        "roofline": {"kernel": dkdv_label(w),
                     "bound": "mfma", "achieved": round(dkdv_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dkdv_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "traffic_unit": "HBM bytes per stage (FETCH_SIZE x2 + WRITE_SIZE x1, "
                                     "copy-calibrated, both kernels)"},
        "memory": {"peak_above_inputs_bytes": int(peak_mem), "resident_bytes": int(resident),
                   "inputs_bytes": int(mem0)},
        "wall_s_timed": round(wall, 3),
        "runs": runs_summary(r, f_fwd, f_bwd, tf),
        "clock": clock_summary(r["clock"], value),
    }
    if not a.no_gemm_reference:
        try:
            g_ms, g_tf = gemm_reference(dev)
        except Exception as e:   # context only: never lose the bench line over it
            g_ms, g_tf = None, None
            out["platform_gemm"] = {"error": f"{type(e).__name__}: {e}"}
    if not a.no_gemm_reference and g_tf:
        out["platform_gemm"] = {
            "what": "8192^3 bf16 GEMM through the vendor BLAS (torch.matmul) on this box, timed after "
                    "the attention steps (median of 5 runs of 60): the practical dense-MFMA rate, "
                    "context only",
            "ms": round(g_ms, 4), "tflops": round(g_tf, 1),
            "pct_of_peak": round(100 * g_tf / PEAK_BF16_TFLOPS, 2),
            "fwd_over_gemm": round(tf(f_fwd, fwd_med) / g_tf, 3),
            "dkdv_over_gemm": round(dkdv_tf / g_tf, 3),
            "step_over_gemm": round(value / g_tf, 3)}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, do, a.cpu_heads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
