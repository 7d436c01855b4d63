"""Attention fwd+bwd throughput on one MI355X, against the bf16 MFMA peak.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]

A step is one forward (fa_fwd) plus one backward (fa_bwd) over the
workload's synthetic inputs, already resident in HBM.  Work is counted on
allowed (query, key) pairs only: 4*D flop per pair forward, 10*D backward
(the five contractions QK^T, PV, dO V^T, P^T dO, dS K / dS^T Q), 14*D in all.

Prints one JSON line: the metric, the per-step time, fwd / bwd / fwd+bwd
TFLOP/s and their fraction of the 2516.6 TFLOP/s dense bf16 peak, the
roofline of the dominant kernel (timed with HIP events on the launch
stream), the peak device memory, and the fp64 oracle timed on a bounded
sample of the same workload on the host CPU.
"""
import argparse
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
        causal = int(np.clip(i - w.shift + 1, 0, kvv).sum())
        if w.kind == W.CAUSAL:
            out.append(causal)
        else:
            steps = w.Skv // w.Sq
            out.append(causal + (steps - 1) * min(w.Sq, kvv))
    return out


def flops(w):
    pairs = sum(pair_count(w)) * w.Hq
    return 4 * w.D * pairs, 10 * w.D * pairs


def find_workload(name):
    for w in W.all_workloads():
        if w.name == name:
            return w
    raise SystemExit(f"unknown workload {name}; known: {[w.name for w in W.all_workloads()]}")


def cpu_baseline(w, q, k, v, do, rows):
    """The fp64 oracle on query head 0, rows [Sq - rows, Sq) (the heaviest
    rows of a causal mask), timed on the host; returns the JSON object."""
    from threadpoolctl import threadpool_info
    from oracle import attention_ref
    Sq = w.Sq
    lo = max(0, Sq - rows)
    kvv = None if w.kv_valid is None else list(w.kv_valid)
    args = [x[:1].double().numpy() for x in (q, k, v, do)]
    t0 = time.perf_counter()
    attention_ref(*args, w.kind, w.shift, kvv, w.scale, heads=[0], rows=(lo, Sq))
    sec = time.perf_counter() - t0
    # allowed pairs in the sample (batch 0, one head)
    wi = w.with_(B=1, kv_valid=None if kvv is None else (kvv[0],))
    i = np.arange(lo, Sq, dtype=np.int64)
    cap = w.Sq if w.kind == W.TTT else w.Skv
    n_valid = cap if kvv is None else min(kvv[0], cap)
    if w.kind == W.FULL:
        pairs = (Sq - lo) * n_valid
    else:
        pairs = int(np.clip(i - w.shift + 1, 0, n_valid).sum())
        if w.kind == W.TTT:
            pairs += (w.Skv // w.Sq - 1) * int((i < n_valid).sum())
    del wi
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": 14 * w.D * pairs / sec / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle, fwd+bwd of batch 0, query head 0, rows [{lo}, {Sq}) "
                      f"of {w.name} ({pairs} allowed pairs, {sec:.2f} s, host nproc {os.cpu_count()})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=W.HEADLINE.name)
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="query rows of one head the oracle baseline computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the library is single-GPU; see DESIGN.md for how it would shard)", file=sys.stderr)
        return 2

    import flash_attention_fa_amd as fa
    w = find_workload(a.workload)
    dev = torch.device("cuda", int(os.environ.get("LOCAL_RANK", 0)))
    torch.cuda.set_device(dev)
    q, k, v, do = W.make_inputs(w, seed=0)
    qg, kg, vg, dog = (x.to(dev) for x in (q, k, v, do))
    kvv = W.kv_valid_tensor(w, dev)
    o = torch.empty_like(qg)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    ws = torch.empty(max(1, fa.fa_bwd_workspace_bytes(qg, kg)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    kw = dict(mask_kind=w.kind, causal_shift=w.shift, kv_valid=kvv, scale=w.scale, stream=stream)

    def fwd():
        fa.fa_fwd(qg, kg, vg, out=o, lse=lse, **kw)

    def bwd():
        fa.fa_bwd(qg, kg, vg, o, lse, dog, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    for _ in range(a.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        ev[s][0].record(stream)
        fwd()
        ev[s][1].record(stream)
        bwd()
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    total_ms = ev[0][0].elapsed_time(ev[-1][2])
    ms_step = total_ms / a.steps
    f_fwd, f_bwd = flops(w)
    fwd_med, bwd_med = float(np.median(fwd_ms)), float(np.median(bwd_ms))
    fwd_avg = float(np.mean(fwd_ms))
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    value = tf(f_fwd + f_bwd, ms_step)
    peak_mem = torch.cuda.max_memory_allocated(dev)
    # inputs + outputs + workspace resident during the step
    resident = sum(t.numel() * t.element_size() for t in (qg, kg, vg, dog, o, lse, dq, dk, dv, ws))

    fwd_tf = tf(f_fwd, fwd_avg)
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
        "roofline": {"kernel": "fwd_kernel (fa_fwd: one launch)", "bound": "mfma",
                     "achieved": round(fwd_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "memory": {"peak_allocated_bytes": int(peak_mem), "resident_bytes": int(resident),
                   "baseline_bytes": int(mem0)},
        "wall_s_timed": round(wall, 3),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, do, a.cpu_rows)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
