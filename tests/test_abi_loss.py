"""The loss entry points of the C ABI on the CPU: struct layout and argument
validation (no kernel runs; fake aligned device addresses are never
dereferenced, and a valid request without a GPU fails with FA_ERR_HIP).

Requests that pass validation would launch on the fake addresses where a GPU
is present, so the tests that make them are marked ``no_device`` and skipped
there; the error paths, which return before any launch, run everywhere."""
import ctypes

import pytest

from flash_attention_fa_amd import _lib


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


no_device = pytest.mark.skipif(_gpu_present(), reason="a valid request on fake addresses would launch")

BASE = 1 << 32
GAP = 1 << 28


def args(N=4, V=100, ss=None):
    a = _lib.fa_lsm_loss_args()
    a.N, a.V = N, V
    a.logits, a.logits_ss = BASE, ss or 128
    a.target, a.target_ss = BASE + GAP, ss or 128
    a.mask = None
    a.m, a.d, a.tsum = BASE + 2 * GAP, BASE + 3 * GAP, BASE + 4 * GAP
    a.row_loss, a.loss, a.grad_loss = BASE + 5 * GAP, BASE + 6 * GAP, BASE + 7 * GAP
    return a


def fwd(a):
    st = _lib.lib().fa_lsm_loss_fwd(ctypes.byref(a) if a is not None else None, None)
    return st, _lib.last_error()


def bwd(a):
    st = _lib.lib().fa_lsm_loss_bwd(ctypes.byref(a) if a is not None else None, None)
    return st, _lib.last_error()


def test_struct_layout():
    assert _lib.fa_lsm_loss_args.logits.offset == 8
    assert _lib.fa_lsm_loss_args.target.offset == 24
    assert _lib.fa_lsm_loss_args.grad_loss.offset == 88
    assert ctypes.sizeof(_lib.fa_lsm_loss_args) == 96


@no_device
def test_valid_request_without_gpu_fails_cleanly():
    for f in (fwd, bwd):
        st, msg = f(args())
        assert st == _lib.FA_ERR_HIP, msg


def test_null_and_size_errors():
    assert fwd(None)[0] == _lib.FA_ERR_INVALID_ARG
    assert bwd(None)[0] == _lib.FA_ERR_INVALID_ARG
    for f in (fwd, bwd):
        a = args(N=-1)
        assert f(a)[0] == _lib.FA_ERR_INVALID_ARG
        a = args(V=0)
        assert f(a)[0] == _lib.FA_ERR_INVALID_ARG
        for field in ("logits", "target", "m", "d", "tsum"):
            a = args()
            setattr(a, field, None)
            st, msg = f(a)
            assert st == _lib.FA_ERR_INVALID_ARG and "NULL" in msg, (field, msg)
    a = args()
    a.row_loss = None
    assert fwd(a)[0] == _lib.FA_ERR_INVALID_ARG
    a = args()
    a.loss = None
    assert fwd(a)[0] == _lib.FA_ERR_INVALID_ARG
    a = args()
    a.grad_loss = None
    assert bwd(a)[0] == _lib.FA_ERR_INVALID_ARG
    # row stride below V: rows would overlap
    a = args(V=100, ss=96)
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_INVALID_ARG and "stride" in msg


@no_device
def test_unaligned_rows_are_accepted():
    for f in (fwd, bwd):
        a = args()
        a.logits = BASE + 4           # 4-byte aligned: accepted
        assert f(a)[0] == _lib.FA_ERR_HIP
        a = args(ss=130)              # any row stride >= V is accepted
        assert f(a)[0] == _lib.FA_ERR_HIP


def test_alignment_errors():
    for f in (fwd, bwd):
        a = args()
        a.logits = BASE + 1
        assert f(a)[0] == _lib.FA_ERR_ALIGNMENT
        a = args()
        a.target = BASE + GAP + 2
        assert f(a)[0] == _lib.FA_ERR_ALIGNMENT
        a = args()
        a.m = BASE + 2 * GAP + 2
        assert f(a)[0] == _lib.FA_ERR_ALIGNMENT
        a = args()
        a.mask = BASE + 9 * GAP + 1
        assert f(a)[0] == _lib.FA_ERR_ALIGNMENT


def test_alias_errors():
    a = args()
    a.m = BASE + 16               # inside the logits
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_ALIAS, msg
    a = args()
    a.row_loss = a.d              # two outputs on one buffer
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_ALIAS, msg
    a = args()
    a.loss = a.target             # the scalar on the target
    assert fwd(a)[0] == _lib.FA_ERR_ALIAS
    a = args()
    a.target = a.logits           # the gradient's buffer is also an input
    st, msg = bwd(a)
    assert st == _lib.FA_ERR_ALIAS, msg
    a = args()
    a.grad_loss = BASE + 32       # upstream gradient inside the logits
    assert bwd(a)[0] == _lib.FA_ERR_ALIAS


def test_empty_rows_backward_is_a_noop():
    # N = 0: the backward has nothing to do and returns before any launch
    assert bwd(args(N=0))[0] == _lib.FA_OK


@no_device
def test_empty_rows_forward_needs_a_device():
    # N = 0: the forward still writes loss = 0, so it needs a device
    assert fwd(args(N=0))[0] == _lib.FA_ERR_HIP
