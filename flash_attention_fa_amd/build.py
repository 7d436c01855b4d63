"""Builds libfa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m flash_attention_fa_amd.build [--jobs N]

Every HIP source is compiled with hipcc for gfx950 only; packed-fp32 VALU
instructions are disabled (-packed-fp32-ops) and no fast-math flags are used,
because the kernels rely on IEEE infinities for masked scores.
"""
import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_f32.hip", "fa_loss.hip"]
HEADERS = ["fa_internal.h", "fa_device.h"]

# Per-source code-generation options (none at present).
EXTRA_FLAGS = {}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = ("packed-fp32-ops", "unknown target feature", "warning generated")
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if ln.strip() and not any(n in ln for n in noise)]
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(msgs))
    return obj, msgs


def build(jobs=4, verbose=False):
    """Compile every source and link libfa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (_, msgs), src in zip(results, SOURCES):
            for m in msgs:
                print(f"[{src}] {m}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libfa.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    path = build(a.jobs, a.verbose)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
