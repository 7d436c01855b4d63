"""The gfx950 lane maps stated in fa_device.h, pinned by single-wave probes
(tests/probe/lane_probe.hip, which calls the header's helpers as the kernels
do).  What each probe must return follows from the stated map alone:

  * mfma32: with the A, B and C lane maps as stated, C0 + A B comes out
    exactly (small integers: every product and sum is exact in fp32).  The
    reduction index k is only defined up to one permutation shared by A and
    B, which is all the kernels rely on (they pair A and B element by element);
    the row and column maps are pinned exactly (a transposed or shifted map
    puts values in the wrong place).
  * lds_read_tr4 on a tile stored at swz_off<D>: reading every 4x16 block with
    the stated per-lane addresses returns the tile transposed, for each D the
    kernels use (this also pins that swz<D> permutes a row's chunks and that a
    4-element read never straddles two of them).
  * half_swap_max / half_swap_sum: lane l gets max / sum of lanes l and l ^ 32.
  * the asynchronous copies: lane l's 16 bytes land at slot l of the LDS block,
    in the per-lane address form and the scalar-base form alike.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "probe", "liblane_probe.so")
SYMBOLS = ("probe_mfma", "probe_tr", "probe_swap", "probe_dma")


def lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (python tests/probe/build_probe.py)")
    L = ctypes.CDLL(LIB)
    P, S = ctypes.c_void_p, ctypes.c_void_p
    L.probe_mfma.argtypes = [P, P, P, P, S]
    L.probe_tr.argtypes = [P, P, ctypes.c_int, S]
    L.probe_swap.argtypes = [P, P, P, S]
    L.probe_dma.argtypes = [P, ctypes.c_uint, P, P, S]
    for f in SYMBOLS:
        getattr(L, f).restype = ctypes.c_int
    return L


def test_probe_library_exports():
    L = ctypes.CDLL(LIB)
    for f in SYMBOLS:
        assert hasattr(L, f), f


def say(msg):
    print(msg, flush=True)


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def run(rc):
    assert rc == 0, f"probe launch returned {rc}"
    torch.cuda.synchronize()


@pytest.mark.gpu
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mfma_lane_map(seed):
    say(f"probe mfma32 seed={seed}")
    rng = np.random.default_rng(seed)
    A = rng.integers(-8, 9, (32, 16)).astype(np.float32)
    B = rng.integers(-8, 9, (16, 32)).astype(np.float32)
    C0 = rng.integers(-100, 101, (32, 32)).astype(np.float32)
    dA = torch.from_numpy(A).to(torch.bfloat16).cuda()
    dB = torch.from_numpy(B).to(torch.bfloat16).cuda()
    dC0 = torch.from_numpy(C0).cuda()
    dC = torch.full((32, 32), float("nan"), device="cuda")
    run(lib().probe_mfma(ptr(dA), ptr(dB), ptr(dC0), ptr(dC), stream()))
    assert np.array_equal(dC.cpu().numpy(), C0 + A @ B)


@pytest.mark.gpu
def test_mfma_lane_map_single_entries():
    # one nonzero in A and one in B: C holds one nonzero, at (row of A,
    # column of B), whatever the k permutation is
    say("probe mfma32 unit entries")
    L = lib()
    rng = np.random.default_rng(7)
    for _ in range(8):
        m, n, k = rng.integers(0, 32), rng.integers(0, 32), rng.integers(0, 16)
        A = np.zeros((32, 16), np.float32)
        B = np.zeros((16, 32), np.float32)
        A[m, k], B[k, n] = 3.0, 5.0
        dA = torch.from_numpy(A).to(torch.bfloat16).cuda()
        dB = torch.from_numpy(B).to(torch.bfloat16).cuda()
        dC0 = torch.zeros(32, 32, device="cuda")
        dC = torch.full((32, 32), float("nan"), device="cuda")
        run(L.probe_mfma(ptr(dA), ptr(dB), ptr(dC0), ptr(dC), stream()))
        want = np.zeros((32, 32), np.float32)
        want[m, n] = 15.0
        assert np.array_equal(dC.cpu().numpy(), want), (m, n, k)


@pytest.mark.gpu
@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_transposing_read_on_swizzled_tile(D):
    say(f"probe lds_read_tr4 on a swizzled [64][{D}] tile")
    # every element a distinct bit pattern (0x4000 + its index: normal, finite
    # bf16 values); the probe only moves bits
    idx = (0x4000 + np.arange(64 * D)).reshape(64, D).astype(np.int16)
    X = torch.from_numpy(idx).view(torch.bfloat16).cuda()
    XT = torch.zeros(D, 64, dtype=torch.int16, device="cuda")
    run(lib().probe_tr(ptr(X), ptr(XT), D, stream()))
    assert np.array_equal(XT.cpu().numpy(), idx.T)


@pytest.mark.gpu
def test_half_swap():
    say("probe half_swap_max / half_swap_sum")
    rng = np.random.default_rng(3)
    x = rng.standard_normal(64).astype(np.float32)
    x[5], x[37] = -np.inf, 2.0
    dx = torch.from_numpy(x).cuda()
    mx = torch.empty(64, device="cuda")
    sm = torch.empty(64, device="cuda")
    run(lib().probe_swap(ptr(dx), ptr(mx), ptr(sm), stream()))
    other = x[np.arange(64) ^ 32]
    assert np.array_equal(mx.cpu().numpy(), np.maximum(x, other))
    assert np.array_equal(sm.cpu().numpy(), x + other)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", [0, 1])
def test_async_copy_landing_slots(seed):
    say(f"probe asynchronous copies seed={seed}")
    n = 300
    rng = np.random.default_rng(seed)
    g = torch.from_numpy(rng.integers(0, 256, 16 * n).astype(np.uint8)).cuda()
    perm = rng.integers(0, n, 128).astype(np.uint32)
    dperm = torch.from_numpy(perm.view(np.int32)).cuda()
    out = torch.zeros(2048, dtype=torch.uint8, device="cuda")
    run(lib().probe_dma(ptr(g), n, ptr(dperm), ptr(out), stream()))
    chunks = g.cpu().numpy().reshape(n, 16)
    assert np.array_equal(out.cpu().numpy().reshape(128, 16), chunks[perm])
