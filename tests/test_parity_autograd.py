"""GPU parity of the autograd drop-in ``attention()`` against the fp64 oracle.

CS336 "Flash Attention (Triton)" offers its kernel as an autograd function
usable in place of the explicit chain; ``attention()`` is that function here:
its forward saves O and LSE, and its backward runs the library's backward.
These cases drive it through ``torch.autograd`` with the layouts a model
hands it: Q, K, V as [B, H, S, D] views of [B, S, H, D] storage (BSHD, no
copy), grouped-query heads, an upstream gradient that is itself a strided
view (one with unit D stride, one without), and the window, frozen-prefix and
TTT masks.  Tolerances are the bf16 bars of the other parity tests.
"""
import numpy as np
import pytest
import torch

import flash_attention_fa_amd as fa
import workloads as W
from oracle import allowed, attention_ref
from parity_util import TOL_BF16, say

pytestmark = pytest.mark.gpu


def bshd_leaf(B, S, H, D, g):
    """A [B, S, H, D] bf16 leaf on the GPU and its [B, H, S, D] view."""
    x = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).cuda().requires_grad_(True)
    return x, x.transpose(1, 2)


def run_case(B, Hq, Hkv, Sq, Skv, D, kind, seed, shift=0, window=None, frozen=0, do_layout="bshd"):
    label = f"autograd kind={kind} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} D={D} shift={shift} " \
            f"window={window} frozen={frozen} dO={do_layout}"
    say(f"[parity] {label}")
    g = torch.Generator("cpu").manual_seed(seed)
    ql, q = bshd_leaf(B, Sq, Hq, D, g)
    kl, k = bshd_leaf(B, Skv, Hkv, D, g)
    vl, v = bshd_leaf(B, Skv, Hkv, D, g)
    assert not q.is_contiguous() and not k.is_contiguous()
    do_cpu = torch.randn(B, Sq, Hq, D, generator=g).to(torch.bfloat16)
    if do_layout == "bshd":          # unit D stride, strided heads and rows
        do = do_cpu.cuda().transpose(1, 2)
    else:                            # D stride 2: the binding must make it contiguous
        wide = torch.zeros(B, Hq, Sq, 2 * D, dtype=torch.bfloat16)
        wide[..., ::2] = do_cpu.transpose(1, 2)
        do = wide.cuda()[..., ::2]
        assert do.stride(-1) == 2
    o = fa.attention(q, k, v, mask_kind=kind, causal_shift=shift, window=window, frozen_keys=frozen)
    assert o.shape == (B, Hq, Sq, D) and o.requires_grad
    o.backward(do)
    torch.cuda.synchronize()
    got = {"O": o.detach(), "dQ": ql.grad.transpose(1, 2), "dK": kl.grad.transpose(1, 2),
           "dV": vl.grad.transpose(1, 2)}
    got = {n: t.float().cpu().numpy().astype(np.float64) for n, t in got.items()}
    to64 = lambda t: t.detach().transpose(1, 2).float().cpu().numpy().astype(np.float64)
    ref = attention_ref(to64(ql), to64(kl), to64(vl), do_cpu.transpose(1, 2).double().numpy(), kind, shift,
                        None, None, window=window)
    A = allowed(kind, Sq, Skv, shift, None, window=window)
    rows, keys = A.any(1), A.any(0)
    keys[:frozen] = False
    errs = {}
    for name in ("O", "dQ", "dK", "dV"):
        gv, rv = got[name], ref[name]
        sel = keys if name in ("dK", "dV") else rows
        assert np.isfinite(gv).all(), f"{label} {name}: non-finite"
        assert np.all(gv[:, :, ~sel] == 0.0), f"{label} {name}: non-zero where nothing is attended or frozen"
        diff = np.abs(gv[:, :, sel] - rv[:, :, sel]).max()
        errs[name] = float(diff / np.abs(rv[:, :, sel]).max())
        assert errs[name] <= TOL_BF16[name], f"{label} {name}: rel err {errs[name]:.3e}"
    say(f"[parity] {label} ok {errs}")


def test_autograd_gqa_causal_bshd_views():
    run_case(2, 8, 2, 300, 300, 128, W.CAUSAL, seed=501)


def test_autograd_do_without_unit_stride():
    run_case(1, 4, 4, 190, 190, 64, W.CAUSAL, seed=502, do_layout="strided_d")


def test_autograd_window():
    run_case(2, 8, 2, 333, 333, 64, W.WINDOW, seed=503, window=(90, 17), shift=1)


def test_autograd_frozen_prefix():
    P = 150
    run_case(1, 8, 2, 260, 260 + P, 128, W.CAUSAL, seed=504, shift=-P, frozen=P)


def test_autograd_ttt():
    run_case(1, 8, 2, 200, 600, 128, W.TTT, seed=505)


def test_autograd_fp32():
    g = torch.Generator("cpu").manual_seed(506)
    q, k, v, do = (torch.randn(1, 2, 70, 32, generator=g) for _ in range(4))
    qg, kg, vg = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o = fa.attention(qg, kg, vg, mask_kind=W.CAUSAL)
    o.backward(do.cuda())
    ref = attention_ref(*(x.double().numpy() for x in (q, k, v, do)), W.CAUSAL)
    for name, t in (("O", o.detach()), ("dQ", qg.grad), ("dK", kg.grad), ("dV", vg.grad)):
        err = float(np.abs(t.double().cpu().numpy() - ref[name]).max())
        assert err <= 1e-4, f"fp32 autograd {name}: {err:.2e}"
