"""The kernels' tile classifier against the oracle's mask predicate, on the CPU.

The attention kernels never look at a (query, key) pair the analytic tile
classifier of fa_device.h rules out: a SKIP tile is not computed, a FULL tile
is computed without a mask, the tile walk visits only the tiles it lists,
rows from ``full_tiles_below`` on see whole leading tiles without
classification, and the dK/dV kernels visit only the query rows of
``query_hull``.  ``tests/host/tile_classifier.cpp`` compiles those helpers
for the host; this test enumerates every pair of small masks of every kind
(ragged sizes, shifts, padding, windows, TTT with several steps) and checks,
against ``oracle.allowed`` (SpecForge page, section Flex Attention; the
WINDOW band):

* no allowed pair sits in a SKIP tile, every pair of a FULL tile is allowed;
* the walk visits every tile that holds an allowed pair, in increasing
  order, each once;
* the leading ``full_tiles_below(qa)`` tiles are entirely allowed for every
  row from qa on;
* every row that attends a key of a block lies inside the block's hull;
* the causal view the bf16 kernels take of a TTT mask covers exactly its
  step-0 part, and the rest of the TTT mask is the one key s*L + i per later
  step s for rows i below kv_valid (the keys ttt_fold and ttt_dkdv_kernel
  take one by one).
"""
import itertools
import os
import subprocess

import numpy as np
import pytest

from oracle import CAUSAL, FULL, TTT, WINDOW, allowed

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "tile_classifier.cpp")
ROOT = os.path.dirname(HERE)
SKIP_, FULL_, PART_ = 0, 1, 2


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    from flash_attention_fa_amd.build import hipcc
    exe = str(tmp_path_factory.mktemp("tile_classifier") / "tile_classifier")
    cmd = [hipcc(), "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "flash_attention_fa_amd", "csrc"),
           SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def cases():
    out = []
    tiles = [(32, 32, 32), (64, 64, 256), (256, 64, 256), (64, 32, 32)]
    for Sq, Skv in [(1, 1), (7, 7), (64, 64), (100, 130), (130, 100), (200, 200)]:
        # negative shifts: a prefix of -shift keys before the diagonal
        for shift, kv in itertools.product((0, 1, 5, 70, -1, -30, -64, -300), (None, 0, 1, 61)):
            for TQ, TK, TKW in tiles:
                kvv = Skv if kv is None else min(kv, Skv)
                out.append((FULL, Sq, Skv, 0, kvv, 0, 0, TQ, TK, TKW, 0))
                out.append((CAUSAL, Sq, Skv, shift, kvv, 0, 0, TQ, TK, TKW, 0))
                for wl, wr in ((0, 0), (3, 0), (0, 5), (17, 9), (200, 200)):
                    out.append((WINDOW, Sq, Skv, shift, kvv, wl, wr, TQ, TK, TKW, 0))
    for L, n in [(1, 2), (7, 3), (40, 2), (64, 3), (100, 3), (130, 2)]:
        for shift, kv in itertools.product((0, 2), (None, 0, 1, 33)):
            for TQ, TK, TKW in tiles:
                kvv = L if kv is None else min(kv, L)
                for view in (0, 1):
                    out.append((TTT, L, n * L, shift, kvv, 0, 0, TQ, TK, TKW, view))
    return out


def run(driver, cs):
    inp = "\n".join(" ".join(str(x) for x in c) for c in cs) + "\n"
    r = subprocess.run([driver], input=inp, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    res, cur = [], None
    for line in r.stdout.splitlines():
        f = line.split()
        if f[0] == "C":
            cur = {"S": {}, "W": {}, "F": {}, "H": {}}
            res.append(cur)
        elif f[0] in "SW":
            cur[f[0]][int(f[1])] = [int(x) for x in f[2:]]
        elif f[0] == "F":
            cur["F"][int(f[1])] = int(f[2])
        else:
            cur["H"][int(f[1])] = (int(f[2]), int(f[3]))
    assert len(res) == len(cs)
    return res


def predicate(c):
    kind, Sq, Skv, shift, kvv, wl, wr, TQ, TK, TKW, view = c
    A = allowed(kind, Sq, Skv, shift, kvv, window=(wl, wr))
    if view == 1:
        # the bf16 kernels' tile loops: TTT's step-0 keys, as a causal mask
        step0 = allowed(CAUSAL, Sq, min(Skv, Sq), shift, kvv)
        assert np.array_equal(A[:, :Sq], step0)
        later = A[:, Sq:]
        i = np.arange(Sq)[:, None]
        j = np.arange(Sq, Skv)[None, :]
        assert np.array_equal(later, ((j % Sq) == i) & (i < kvv)), "TTT beyond step 0 is one key per step"
        return step0
    return A


def test_tile_classifier_against_the_predicate(driver):
    cs = cases()
    res = run(driver, cs)
    checked = 0
    for c, r in zip(cs, res):
        A = predicate(c)
        Sq, nk = A.shape
        TQ, TK, TKW = c[7], c[8], c[9]
        ntk = -(-c[2] // TK)
        for qa in range(0, Sq, TQ):
            qb = min(Sq, qa + TQ)
            states = r["S"][qa]
            assert len(states) == ntk
            need = set()
            for t, st in enumerate(states):
                sub = A[qa:qb, t * TK:min(nk, t * TK + TK)]
                if st == SKIP_:
                    assert not sub.any(), (c, qa, t, "allowed pair in a SKIP tile")
                elif st == FULL_:
                    assert t * TK + TK <= nk and sub.all(), (c, qa, t, "FULL tile with a masked pair")
                if sub.any():
                    need.add(t)
            walk = r["W"][qa]
            assert walk == sorted(set(walk)), (c, qa, "walk not increasing or repeats a tile")
            assert need <= set(walk), (c, qa, "walk misses a tile with allowed pairs", sorted(need - set(walk)))
            assert all(0 <= t < -(-nk // TK) for t in walk), (c, qa, "walk leaves the key range")
            f = r["F"][qa]
            assert f * TK <= nk and A[qa:, :f * TK].all(), (c, qa, f, "full_tiles_below too large")
            checked += 1
        for k0 in range(0, c[2], TKW):
            lo, hi = r["H"][k0]
            rows = np.nonzero(A[:, k0:min(nk, k0 + TKW)].any(1))[0] if k0 < nk else np.array([], int)
            if len(rows):
                assert lo <= rows.min() and rows.max() < hi, (c, k0, lo, hi, "row outside the hull")
    assert checked > 1000
