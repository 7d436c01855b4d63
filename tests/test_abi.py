"""The C ABI on the CPU: symbols, struct layout and argument validation.

No kernel runs here.  Validation happens before any HIP call, so fake
(aligned, never dereferenced) device addresses exercise every error path; a
valid request on a machine without a GPU must fail cleanly with FA_ERR_HIP.

A request that passes validation would launch kernels on those fake
addresses where a GPU is present, so every test that builds one is marked
``no_device`` and skipped there; the error paths, which return before any
launch, run everywhere.
"""
import ctypes
import os
import re

import pytest

from flash_attention_fa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
BASE = 1 << 32          # fake device addresses: 16-byte aligned, far apart
GAP = 1 << 28


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:fa_status|size_t|const char\*)\s+(fa_\w+)\s*\(",
                                 src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n), n


def _c_layout(structs):
    """sizeof and offsetof of every field, as gcc lays out include/fa.h."""
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(HERE)
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "fa.h"', 'int main(void) {']
    for name, fields in structs.items():
        lines.append(f'  printf("{name} sizeof %zu\\n", sizeof({name}));')
        for f in fields:
            lines.append(f'  printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines += ['  return 0;', '}']
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        with open(src, "w") as f:
            f.write("\n".join(lines) + "\n")
        subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
                        "-I", "/opt/rocm/include", src, "-o", exe], check=True, capture_output=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return {tuple(l.split()[:2]): int(l.split()[2]) for l in out.splitlines()}


def test_struct_layout_matches_header():
    # every ctypes mirror against the layout gcc gives the structs of fa.h
    structs = {"fa_tensor": _lib.fa_tensor, "fa_mask_desc": _lib.fa_mask_desc,
               "fa_fwd_args": _lib.fa_fwd_args, "fa_bwd_args": _lib.fa_bwd_args,
               "fa_lsm_loss_args": _lib.fa_lsm_loss_args}
    c = _c_layout({n: [f[0] for f in t._fields_] for n, t in structs.items()})
    for n, t in structs.items():
        assert c[(n, "sizeof")] == ctypes.sizeof(t), n
        for f in t._fields_:
            assert c[(n, f[0])] == getattr(t, f[0]).offset, (n, f[0])


def _t(slot, B, H, S, D, eb=2, strides=None):
    st = strides or (H * S * D, S * D, D)
    return _lib.fa_tensor(BASE + slot * GAP, *st)


def fwd_args(B=1, Hq=4, Hkv=2, Sq=64, Skv=64, D=64, dtype=_lib.FA_BF16, kind=1, shift=0, window=(0, 0),
             frozen=0):
    a = _lib.fa_fwd_args()
    a.dtype, a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = dtype, B, Hq, Hkv, Sq, Skv, D
    a.scale = 0.0
    a.q, a.k, a.v, a.o = _t(0, B, Hq, Sq, D), _t(1, B, Hkv, Skv, D), _t(2, B, Hkv, Skv, D), _t(3, B, Hq, Sq, D)
    a.lse = BASE + 4 * GAP
    a.mask = _lib.fa_mask_desc(kind, shift, None, *window, frozen)
    return a


def bwd_args(B=1, Hq=4, Hkv=2, Sq=64, Skv=64, D=64, dtype=_lib.FA_BF16, kind=1):
    a = _lib.fa_bwd_args()
    a.dtype, a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = dtype, B, Hq, Hkv, Sq, Skv, D
    a.scale = 0.0
    a.q, a.k, a.v = _t(0, B, Hq, Sq, D), _t(1, B, Hkv, Skv, D), _t(2, B, Hkv, Skv, D)
    a.o, a.dout = _t(3, B, Hq, Sq, D), _t(4, B, Hq, Sq, D)
    a.lse = BASE + 5 * GAP
    a.dq, a.dk, a.dv = _t(6, B, Hq, Sq, D), _t(7, B, Hkv, Skv, D), _t(8, B, Hkv, Skv, D)
    a.mask = _lib.fa_mask_desc(kind, 0, None)
    return a


WS = BASE + 9 * GAP


def fwd(a, ws=WS, ws_bytes=1 << 24):
    st = _lib.lib().fa_fwd(a, ws, ws_bytes, None)
    return st, _lib.last_error()


def bwd(a, ws=WS, ws_bytes=1 << 20):
    st = _lib.lib().fa_bwd(a, ws, ws_bytes, None)
    return st, _lib.last_error()


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Requests that pass validation reach a launch when a device exists: with the
# fake addresses above that would be a memory fault, so they run only where
# there is no GPU (and must then stop at FA_ERR_HIP).
no_device = pytest.mark.skipif(_gpu_present(), reason="a valid request on fake addresses would launch")


@no_device
def test_valid_request_without_device_fails_cleanly():
    st, msg = fwd(fwd_args())
    assert st == _lib.FA_ERR_HIP and "device" in msg
    st, msg = bwd(bwd_args())
    assert st == _lib.FA_ERR_HIP and "device" in msg


FWD_CASES = [
    ("bad D", dict(D=48), _lib.FA_ERR_UNSUPPORTED, "head dim"),
    ("bad D 256", dict(D=256), _lib.FA_ERR_UNSUPPORTED, "head dim"),
    ("bad dtype", dict(dtype=7), _lib.FA_ERR_UNSUPPORTED, "dtype"),
    ("bad kind", dict(kind=5), _lib.FA_ERR_UNSUPPORTED, "mask kind"),
    ("gqa not dividing", dict(Hq=6, Hkv=4), _lib.FA_ERR_INVALID_ARG, "multiple of Hkv"),
    ("zero heads", dict(Hq=0), _lib.FA_ERR_INVALID_ARG, "non-positive"),
    ("negative S", dict(Sq=-1), _lib.FA_ERR_INVALID_ARG, "negative size"),
    ("negative shift with TTT", dict(kind=2, Sq=64, Skv=128, shift=-2), _lib.FA_ERR_INVALID_ARG, "causal_shift"),
    ("negative frozen_keys", dict(frozen=-1), _lib.FA_ERR_INVALID_ARG, "frozen_keys"),
    ("ttt skv not multiple", dict(kind=2, Sq=64, Skv=100), _lib.FA_ERR_INVALID_ARG, "multiple of Sq"),
    ("negative window", dict(kind=3, window=(4, -1)), _lib.FA_ERR_INVALID_ARG, "negative window"),
]


@no_device
def test_prefix_masks_are_accepted():
    # a negative shift (a prefix before the diagonal) with CAUSAL and WINDOW,
    # and frozen keys, pass validation (and fail only for want of a device)
    for kw in (dict(kind=1, shift=-16, Skv=80), dict(kind=3, shift=-4, window=(8, 0)),
               dict(kind=1, shift=-16, Skv=80, frozen=16)):
        st, msg = fwd(fwd_args(**kw))
        assert st == _lib.FA_ERR_HIP, (kw, msg)


@pytest.mark.parametrize("name,kw,status,text", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_validation(name, kw, status, text):
    st, msg = fwd(fwd_args(**kw))
    assert st == status, msg
    assert text in msg


def test_forward_pointer_alignment_alias_and_null():
    a = fwd_args()
    a.q.data = BASE + 8                       # misaligned base
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_ALIGNMENT and "q" in msg
    a = fwd_args()
    a.k.stride_s = 60                         # 120 bytes: not a multiple of 16
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_ALIGNMENT and "k" in msg
    a = fwd_args()
    a.o.data = a.q.data + 64                  # output inside an input
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_ALIAS
    a = fwd_args()
    a.lse = a.v.data                          # lse on top of v
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_ALIAS and "lse" in msg
    a = fwd_args()
    a.v.data = None
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_INVALID_ARG and "NULL" in msg
    a = fwd_args()
    a.lse = None
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_INVALID_ARG and "lse" in msg
    a = fwd_args()
    a.o.stride_s = 32                         # output rows overlap each other (D = 64)
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_INVALID_ARG and "overlap" in msg
    st = _lib.lib().fa_fwd(None, WS, 1 << 24, None)
    assert st == _lib.FA_ERR_INVALID_ARG


def test_forward_workspace():
    a = fwd_args(B=2, Hkv=2, Skv=100, D=64)
    need = _lib.lib().fa_fwd_workspace_bytes(a)
    # V^T: [B, Hkv, D, Skv rounded up to 64] bfloat16, rounded up to 256 bytes
    assert need == (2 * 2 * 64 * 128 * 2 + 255) // 256 * 256
    assert _lib.lib().fa_fwd_workspace_bytes(None) == 0
    assert _lib.lib().fa_fwd_workspace_bytes(fwd_args(dtype=_lib.FA_F32)) == 0
    a = fwd_args(Skv=64, Sq=64)
    need = _lib.lib().fa_fwd_workspace_bytes(a)
    st, msg = fwd(a, ws_bytes=need - 1)
    assert st == _lib.FA_ERR_INVALID_ARG and "workspace too small" in msg
    st, msg = fwd(a, ws=None)
    assert st == _lib.FA_ERR_INVALID_ARG and "workspace" in msg
    st, msg = fwd(a, ws=WS + 16)
    assert st == _lib.FA_ERR_ALIGNMENT and "workspace" in msg
    st, msg = fwd(a, ws=a.v.data)             # workspace on an input
    assert st == _lib.FA_ERR_ALIAS and "workspace" in msg
    st, msg = fwd(a, ws=a.o.data)             # workspace on the output
    assert st == _lib.FA_ERR_ALIAS and "workspace" in msg
    # key counts whose V^T rows would not fit 32-bit offsets are refused
    st, msg = fwd(fwd_args(B=1, Hq=1, Hkv=1, Sq=64, Skv=1 << 24, kind=0), ws_bytes=1 << 40)
    assert st == _lib.FA_ERR_UNSUPPORTED and "Skv" in msg


@no_device
def test_f32_forward_takes_no_workspace():
    # fp32 needs none: a NULL workspace is accepted (and fails only for want of a device)
    st, msg = fwd(fwd_args(dtype=_lib.FA_F32), ws=None, ws_bytes=0)
    assert st == _lib.FA_ERR_HIP, msg


def test_forward_empty_is_a_noop():
    for kw in (dict(B=0), dict(Sq=0)):
        a = fwd_args(**kw)
        st, msg = fwd(a)
        assert st == _lib.FA_OK, msg


def test_backward_validation():
    a = bwd_args()
    need = _lib.lib().fa_bwd_workspace_bytes(a)
    # Delta and LSE*log2(e) [B, Hq, Sq], then the dK/dV halves' float32 sums 4 x [B, Hkv, Skv, D]
    assert need == 2 * ((1 * 4 * 64 * 4 + 255) // 256 * 256) + 4 * 1 * 2 * 64 * 64 * 4
    assert _lib.lib().fa_bwd_workspace_bytes(None) == 0
    st, msg = bwd(a, ws_bytes=need - 1)
    assert st == _lib.FA_ERR_INVALID_ARG and "workspace too small" in msg
    st, msg = bwd(a, ws=None)
    assert st == _lib.FA_ERR_INVALID_ARG and "workspace" in msg
    st, msg = bwd(a, ws=WS + 16)
    assert st == _lib.FA_ERR_ALIGNMENT and "workspace" in msg
    a = bwd_args()
    a.dk.data = a.dq.data                     # two outputs on one buffer
    st, msg = bwd(a)
    assert st == _lib.FA_ERR_ALIAS
    a = bwd_args()
    a.dv.data = a.dout.data                   # output on an input
    st, msg = bwd(a)
    assert st == _lib.FA_ERR_ALIAS
    st, msg = bwd(bwd_args(), ws=bwd_args().q.data)   # workspace on an input
    assert st == _lib.FA_ERR_ALIAS and "workspace" in msg
    st, msg = bwd(bwd_args(D=8))
    assert st == _lib.FA_ERR_UNSUPPORTED


def test_workspace_is_linear_in_sequence_length():
    sizes = [_lib.lib().fa_bwd_workspace_bytes(bwd_args(B=1, Hq=32, Hkv=4, Sq=s, Skv=s, D=128))
             for s in (16384, 32768)]
    # Delta and LSE*log2(e) [B, Hq, Sq], then the dK/dV halves' float32 sums 4 x [B, Hkv, Skv, D]
    assert sizes[1] == 2 * sizes[0] == 2 * (2 * 32 * 16384 * 4 + 4 * 4 * 16384 * 128 * 4)
    # under TTT only the Sq step-0 keys have partial sums
    ttt = bwd_args(B=1, Hq=32, Hkv=4, Sq=256, Skv=768, D=128, kind=_lib.FA_MASK_TTT)
    assert _lib.lib().fa_bwd_workspace_bytes(ttt) == 2 * 32 * 256 * 4 + 4 * 4 * 256 * 128 * 4
    # bf16 at every head dim holds the partial sums; fp32 needs none
    assert _lib.lib().fa_bwd_workspace_bytes(bwd_args(B=1, Hq=32, Hkv=4, Sq=256, Skv=256, D=64)) == \
        2 * 32 * 256 * 4 + 4 * 4 * 256 * 64 * 4
    assert _lib.lib().fa_bwd_workspace_bytes(bwd_args(B=1, Hq=32, Hkv=4, Sq=256, Skv=256, D=32)) == \
        2 * 32 * 256 * 4 + 4 * 4 * 256 * 32 * 4
    assert _lib.lib().fa_bwd_workspace_bytes(bwd_args(B=1, Hq=32, Hkv=4, Sq=256, Skv=256, D=16)) == \
        2 * 32 * 256 * 4 + 4 * 4 * 256 * 16 * 4
    assert _lib.lib().fa_bwd_workspace_bytes(
        bwd_args(B=1, Hq=32, Hkv=4, Sq=256, Skv=256, D=128, dtype=_lib.FA_F32)) == 2 * 32 * 256 * 4
    sizes = [_lib.lib().fa_fwd_workspace_bytes(fwd_args(B=1, Hq=32, Hkv=4, Sq=s, Skv=s, D=128))
             for s in (16384, 32768)]
    assert sizes[1] == 2 * sizes[0] == 2 * 4 * 128 * 16384 * 2


def test_bwd_stage_rejects_unknown_stage():
    for stage in (-1, 3, 100):
        st = _lib.lib().fa_bwd_stage(bwd_args(), stage, WS, 1 << 20, None)
        assert st == _lib.FA_ERR_INVALID_ARG
        assert "stage" in _lib.last_error()


def test_bwd_stage_validates_like_bwd():
    # the same argument errors come back from every stage, before any launch
    bad = [bwd_args(Hq=3, Hkv=2), bwd_args(D=96), bwd_args(dtype=7)]
    for a in bad:
        ref, _ = bwd(a)
        assert ref != _lib.FA_OK
        for stage in (_lib.FA_BWD_DELTA, _lib.FA_BWD_DKDV, _lib.FA_BWD_DQ):
            assert _lib.lib().fa_bwd_stage(a, stage, WS, 1 << 20, None) == ref
    # workspace too small
    a = bwd_args()
    for stage in (_lib.FA_BWD_DELTA, _lib.FA_BWD_DKDV, _lib.FA_BWD_DQ):
        assert _lib.lib().fa_bwd_stage(a, stage, WS, 16, None) == _lib.FA_ERR_INVALID_ARG


# ---- fa_fwd_noalloc: the forward with the library's static scratch --------

def fwd_noalloc(a):
    st = _lib.lib().fa_fwd_noalloc(a, None)
    return st, _lib.last_error()


def test_noalloc_validates_like_fa_fwd():
    for name, kw, status, text in FWD_CASES:
        st, msg = fwd_noalloc(fwd_args(**kw))
        assert st == status and text in msg, (name, msg)
    assert _lib.lib().fa_fwd_noalloc(None, None) == _lib.FA_ERR_INVALID_ARG
    a = fwd_args()
    a.o.data = a.q.data + 64                  # output inside an input
    assert fwd_noalloc(a)[0] == _lib.FA_ERR_ALIAS
    for kw in (dict(B=0), dict(Sq=0)):        # empty: a no-op
        assert fwd_noalloc(fwd_args(**kw))[0] == _lib.FA_OK


def test_noalloc_refuses_shapes_beyond_its_scratch():
    cap = _lib.FWD_NOALLOC_SCRATCH_BYTES
    # V^T of B*Hkv*D*Skv bf16 values: 64 MiB holds Skv = 65536 at Hkv=4, D=128,
    # and not 65600 (rounded up to 65600 keys, 64.06 MiB)
    ok = fwd_args(B=1, Hq=32, Hkv=4, Sq=64, Skv=65536, D=128, kind=0)
    big = fwd_args(B=1, Hq=32, Hkv=4, Sq=64, Skv=65600, D=128, kind=0)
    assert _lib.lib().fa_fwd_workspace_bytes(ok) == cap
    assert _lib.lib().fa_fwd_workspace_bytes(big) > cap
    st, msg = fwd_noalloc(big)
    assert st == _lib.FA_ERR_UNSUPPORTED and "scratch" in msg and "fa_fwd" in msg


@no_device
def test_noalloc_valid_request_without_device_fails_cleanly():
    st, msg = fwd_noalloc(fwd_args())
    assert st == _lib.FA_ERR_HIP, msg
    # fp32 needs no scratch at any size: never refused for its size
    st, msg = fwd_noalloc(fwd_args(B=1, Hq=32, Hkv=4, Sq=64, Skv=65600, D=128, kind=0, dtype=_lib.FA_F32))
    assert st == _lib.FA_ERR_HIP, msg


# ---- the key bias (fa_mask_desc.key_bias) ----------------------------------

BIAS = BASE + 10 * GAP


def test_key_bias_validation():
    for make, call in ((fwd_args, fwd), (bwd_args, bwd)):
        a = make()
        a.mask.key_bias = BIAS + 2                # not 4-byte aligned
        st, msg = call(a, ws_bytes=1 << 26)
        assert st == _lib.FA_ERR_ALIGNMENT and "key_bias" in msg
        a = make()
        a.mask.key_bias, a.mask.key_bias_stride_b = BIAS, -64
        st, msg = call(a, ws_bytes=1 << 26)
        assert st == _lib.FA_ERR_INVALID_ARG and "key_bias_stride_b" in msg
    # the bias is an input: no output or workspace may overlap it
    a = fwd_args()
    a.mask.key_bias = a.o.data + 256
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_ALIAS and "key_bias" in msg
    a = fwd_args()
    a.mask.key_bias = a.lse
    st, msg = fwd(a)
    assert st == _lib.FA_ERR_ALIAS and "key_bias" in msg
    a = bwd_args()
    a.mask.key_bias = a.dk.data
    st, msg = bwd(a, ws_bytes=1 << 26)
    assert st == _lib.FA_ERR_ALIAS and "dk" in msg
    a = bwd_args()
    a.mask.key_bias = WS + 64                 # inside the workspace
    st, msg = bwd(a, ws_bytes=1 << 26)
    assert st == _lib.FA_ERR_ALIAS and "workspace" in msg
    # empty shapes never read the bias: any pointer passes the bias checks
    a = fwd_args(B=0)
    a.mask.key_bias = BIAS + 2
    assert fwd(a)[0] == _lib.FA_OK


def test_key_bias_workspace_bytes():
    # bf16: the scaled bias copy, float32 [B, Skv rounded up to 64], rounded up
    # to 256 bytes, after the forward's V^T and after the backward's arrays
    for B, Skv in ((1, 64), (2, 100), (3, 1)):
        a = fwd_args(B=B, Skv=Skv)
        base = _lib.lib().fa_fwd_workspace_bytes(a)
        a.mask.key_bias = BIAS
        extra = (B * ((Skv + 63) // 64 * 64) * 4 + 255) // 256 * 256
        assert _lib.lib().fa_fwd_workspace_bytes(a) == base + extra
        b = bwd_args(B=B, Skv=Skv)
        base = _lib.lib().fa_bwd_workspace_bytes(b)
        b.mask.key_bias = BIAS
        assert _lib.lib().fa_bwd_workspace_bytes(b) == base + extra
    # fp32 reads the caller's bias as is: no extra scratch
    for make, f in ((fwd_args, _lib.lib().fa_fwd_workspace_bytes), (bwd_args, _lib.lib().fa_bwd_workspace_bytes)):
        a = make(dtype=_lib.FA_F32)
        base = f(a)
        a.mask.key_bias = BIAS
        assert f(a) == base
    # a workspace sized without the bias is too small with it
    a = fwd_args()
    need = _lib.lib().fa_fwd_workspace_bytes(a)
    a.mask.key_bias = BIAS
    st, msg = fwd(a, ws_bytes=need)
    assert st == _lib.FA_ERR_INVALID_ARG and "workspace too small" in msg


@no_device
def test_key_bias_valid_request_without_device_fails_cleanly():
    for dtype in (_lib.FA_BF16, _lib.FA_F32):
        a = fwd_args(dtype=dtype)
        a.mask.key_bias, a.mask.key_bias_stride_b = BIAS, 0
        st, msg = fwd(a, ws_bytes=1 << 26)
        assert st == _lib.FA_ERR_HIP
        b = bwd_args(dtype=dtype)
        b.mask.key_bias, b.mask.key_bias_stride_b = BIAS, 64
        st, msg = bwd(b, ws_bytes=1 << 26)
        assert st == _lib.FA_ERR_HIP
