"""No kernel writes outside its outputs: every output sits in storage with
sentinel-filled slack, checked bitwise after each call.

Each output of the attention calls (O, LSE, dQ, dK, dV) and of the loss
calls (m, d, tsum, row_loss, loss and the gradient written over the logits)
is carved out of a larger buffer: guard regions before and after it, and for
the [B, H, S, D] tensors a BSHD layout with eight padding columns after every
row (so rows, heads and batches all have gaps between them).  The
workspaces get a guard region after their last byte.  After the calls every
byte of the slack must still hold the sentinel (a NaN bit pattern), and the
attention outputs must be bitwise what the same calls write into plain
contiguous tensors (their arithmetic does not depend on the output layout;
the loss reads strided rows through another load path, so its outputs are
compared to rounding).  The
cases have ragged tails (lengths that are not tile multiples), padded keys,
every mask kind and both the few- and many-workgroup launch shapes.
"""
import numpy as np
import pytest
import torch

import flash_attention_fa_amd as fa
import workloads as W
from parity_util import say

pytestmark = pytest.mark.gpu

GUARD = 4096            # elements of slack before and after each buffer
PAD = 8                 # padding columns after each row of a [B, H, S, D] output
SENT8 = 0xA5            # workspace bytes
SENT16 = 0x7FC1         # a bf16 NaN with a payload
SENT32 = 0x7FC0A5A5     # an fp32 NaN with a payload


def _i32(x):
    return x - (1 << 32) if x >= (1 << 31) else x


def iview(t):
    """t's bits as integers of its element size."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.dtype.itemsize])


def sentinel(dtype):
    return {1: SENT8, 2: SENT16, 4: _i32(SENT32)}[dtype.itemsize]


class Guarded:
    """A buffer of n payload elements with GUARD sentinel elements each side."""

    def __init__(self, n, dtype):
        self.n = n
        self.flat = torch.empty(GUARD + n + GUARD, dtype=dtype, device="cuda")
        iview(self.flat).fill_(sentinel(dtype))

    def payload(self):
        return self.flat[GUARD:GUARD + self.n]

    def guards_intact(self):
        v, sent = iview(self.flat), sentinel(self.flat.dtype)
        return bool((v[:GUARD] == sent).all()) and bool((v[GUARD + self.n:] == sent).all())


def bshd_out(B, H, S, D, dtype=torch.bfloat16):
    """A [B, H, S, D] view of [B, S, H, D + PAD] storage inside a guarded buffer."""
    g = Guarded(B * S * H * (D + PAD), dtype)
    store = g.payload().view(B, S, H, D + PAD)
    return g, store, store[..., :D].transpose(1, 2)


def pads_intact(store, D):
    return bool((iview(store[..., D:].contiguous()) == SENT16).all())


CASES = [
    # name, B, Hq, Hkv, Sq, Skv, D, kind, shift, kv_valid, window
    ("causal_ragged_d128", 2, 4, 2, 300, 300, 128, W.CAUSAL, 0, None, None),
    ("full_kvvalid_d64", 2, 4, 4, 200, 333, 64, W.FULL, 0, (300, 77), None),
    ("ttt_d128", 1, 8, 2, 130, 390, 128, W.TTT, 0, (100,), None),
    ("window_d32", 2, 4, 2, 333, 333, 32, W.WINDOW, 3, (290, 333), (40, 9)),
    ("causal_d16", 2, 4, 2, 257, 257, 16, W.CAUSAL, 1, None, None),
    ("many_wg_ttt_d128", 4, 128, 16, 300, 900, 128, W.TTT, 0, (300, 250, 1, 299), None),
    ("unsplit_causal_d64", 16, 64, 64, 256, 256, 64, W.CAUSAL, 0, None, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_outputs_stay_in_bounds(case):
    name, B, Hq, Hkv, Sq, Skv, D, kind, shift, kvv, win = case
    say(f"[guard] {name}")
    g = torch.Generator("cpu").manual_seed(600 + D)
    mk = lambda H, S: torch.randn(B, H, S, D, generator=g).to(torch.bfloat16).cuda()
    q, k, v, do = mk(Hq, Sq), mk(Hkv, Skv), mk(Hkv, Skv), mk(Hq, Sq)
    kv = None if kvv is None else torch.tensor(kvv, dtype=torch.int32, device="cuda")
    kw = dict(mask_kind=kind, causal_shift=shift, kv_valid=kv, window=win)

    # reference: contiguous outputs allocated by the binding
    o_ref, lse_ref = fa.fa_fwd(q, k, v, **kw)
    dq_ref, dk_ref, dv_ref = fa.fa_bwd(q, k, v, o_ref, lse_ref, do, **kw)

    go, so, o = bshd_out(B, Hq, Sq, D)
    gl = Guarded(B * Hq * Sq, torch.float32)
    lse = gl.payload().view(B, Hq, Sq)
    fws_n = max(1, fa.fa_fwd_workspace_bytes(q, k))
    gfw = Guarded(fws_n + 256, torch.uint8)
    fws = gfw.payload()[:fws_n]
    fa.fa_fwd(q, k, v, out=o, lse=lse, workspace=_aligned(fws), **kw)
    gdq, sdq, dq = bshd_out(B, Hq, Sq, D)
    gdk, sdk, dk = bshd_out(B, Hkv, Skv, D)
    gdv, sdv, dv = bshd_out(B, Hkv, Skv, D)
    bws_n = max(1, fa.fa_bwd_workspace_bytes(q, k, mask_kind=kind))
    gbw = Guarded(bws_n + 256, torch.uint8)
    bws = gbw.payload()[:bws_n]
    fa.fa_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=_aligned(bws), **kw)
    torch.cuda.synchronize()

    for label, gd in (("O", go), ("LSE", gl), ("dQ", gdq), ("dK", gdk), ("dV", gdv),
                      ("fwd workspace", gfw), ("bwd workspace", gbw)):
        assert gd.guards_intact(), f"{name}: write outside {label}"
    for label, gd, st in (("O", go, so), ("dQ", gdq, sdq), ("dK", gdk, sdk), ("dV", gdv, sdv)):
        assert pads_intact(st, D), f"{name}: write into the row padding of {label}"
    # workspace tails (between the size asked for and the guard) untouched too
    for label, gd, n in (("fwd workspace", gfw, fws_n), ("bwd workspace", gbw, bws_n)):
        assert bool((gd.payload()[n:] == SENT8).all()), f"{name}: write past the {label}"
    for label, a, b in (("O", o, o_ref), ("LSE", lse, lse_ref), ("dQ", dq, dq_ref), ("dK", dk, dk_ref),
                        ("dV", dv, dv_ref)):
        assert torch.equal(a, b), f"{name}: {label} differs from the contiguous-output call"


def _aligned(buf):
    """The library asks for 256-byte aligned workspaces; GUARD * 1 byte of
    uint8 slack keeps the payload at the allocation's 256-byte alignment."""
    assert buf.data_ptr() % 256 == 0, "guarded workspace lost its alignment"
    return buf


def test_loss_outputs_stay_in_bounds():
    N, V, pad = 37, 1003, 13            # rows not a multiple of anything, odd row stride
    say("[guard] loss")
    x, t, m = W.make_loss_inputs(W.LossWorkload("guard", 1, N, V), seed=7)
    gx = Guarded(N * (V + pad), torch.float32)
    xs = gx.payload().view(N, V + pad)
    xs[:, :V] = x.cuda()
    logits = xs[:, :V]
    tg, mg = t.cuda(), m.cuda()
    x_ref = x.cuda().clone()
    loss_ref, row_ref, m_ref, d_ref, ts_ref = fa.lsm_loss_fwd(x_ref, tg, mg)
    fa.lsm_loss_bwd(x_ref, tg, mg, m_ref, d_ref, ts_ref, torch.ones(1, device="cuda"))

    import ctypes
    from flash_attention_fa_amd import _lib
    bufs = {nm: Guarded(N if nm != "loss" else 1, torch.float32) for nm in ("m", "d", "tsum", "row_loss", "loss")}
    a = _lib.fa_lsm_loss_args()
    a.N, a.V = N, V
    a.logits, a.logits_ss = logits.data_ptr(), logits.stride(0)
    a.target, a.target_ss = tg.data_ptr(), tg.stride(0)
    a.mask = mg.data_ptr()
    for nm, gb in bufs.items():
        setattr(a, nm, gb.payload().data_ptr())
    stream = torch.cuda.current_stream().cuda_stream
    _lib.check(_lib.lib().fa_lsm_loss_fwd(ctypes.byref(a), stream))
    one = torch.ones(1, device="cuda")
    a.grad_loss = one.data_ptr()
    _lib.check(_lib.lib().fa_lsm_loss_bwd(ctypes.byref(a), stream))
    torch.cuda.synchronize()
    assert gx.guards_intact(), "loss: write outside the logits buffer"
    assert bool((xs[:, V:].contiguous().view(torch.int32) == _i32(SENT32)).all()), "loss: write into row padding"
    for nm, gb in bufs.items():
        assert gb.guards_intact(), f"loss: write outside {nm}"
    # the strided rows take another load path, so compare to rounding, not bitwise
    for nm, ref in (("loss", loss_ref.reshape(1)), ("row_loss", row_ref), ("m", m_ref), ("d", d_ref),
                    ("tsum", ts_ref)):
        torch.testing.assert_close(bufs[nm].payload(), ref, rtol=1e-5, atol=1e-6, msg=nm)
    torch.testing.assert_close(logits, x_ref, rtol=1e-5, atol=1e-7, msg="loss gradient")
