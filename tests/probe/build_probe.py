"""Builds tests/probe/liblane_probe.so, the single-wave probes of the gfx950
building blocks the attention kernels use (test infrastructure), with the
library's own compiler flags.

    python tests/probe/build_probe.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "liblane_probe.so")
SRC = os.path.join(HERE, "lane_probe.hip")


def build():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from flash_attention_fa_amd.build import hipcc, common_flags
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + common_flags() + ["-shared", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the lane probes failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
