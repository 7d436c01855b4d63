"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare with the fp64 oracle on the very same inputs.

Tolerances (per tensor, over rows that have at least one allowed key):
  * float32: max |err| <= 1e-4 on O, LSE, dQ, dK, dV;
  * bfloat16: max|err| / max|ref| <= 2e-2 on O and <= 5e-2 on dQ, dK, dV,
    and max |err| <= 1e-2 on LSE.
Rows with no allowed key must hold exactly O = 0, LSE = 0, dQ = 0, and keys
no query may attend, and frozen keys, must hold exactly dK = dV = 0.  With a
key bias, a key whose bias is -inf counts as not allowed.
"""
import sys

import numpy as np
import torch

import flash_attention_fa_amd as fa
from oracle import allowed, attention_ref

TOL_BF16 = {"O": 2e-2, "dQ": 5e-2, "dK": 5e-2, "dV": 5e-2}
TOL_LSE_BF16 = 1e-2
TOL_F32 = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(q, k, v, do, kind, shift=0, kv_valid=None, scale=None, device="cuda", window=None, frozen=0,
            bias=None):
    """Forward + backward through the library; returns numpy float64 arrays.
    ``bias``: a float32 [B, Skv] tensor (any device) or None."""
    qg, kg, vg, dog = (x.to(device) for x in (q, k, v, do))
    kvv = None if kv_valid is None else torch.tensor(list(kv_valid), dtype=torch.int32, device=device)
    bg = None if bias is None else bias.to(device)
    o, lse = fa.fa_fwd(qg, kg, vg, mask_kind=kind, causal_shift=shift, kv_valid=kvv, scale=scale,
                       window=window, frozen_keys=frozen, key_bias=bg)
    dq, dk, dv = fa.fa_bwd(qg, kg, vg, o, lse, dog, mask_kind=kind, causal_shift=shift,
                           kv_valid=kvv, scale=scale, window=window, frozen_keys=frozen, key_bias=bg)
    torch.cuda.synchronize()
    return dict(O=to_np(o), LSE=to_np(lse), dQ=to_np(dq), dK=to_np(dk), dV=to_np(dv))


def structure(kind, B, Sq, Skv, shift, kv_valid, window=None, bias=None):
    """(nonempty rows [B, Sq], attended keys [B, Skv]) from the oracle's
    predicate (and the finite entries of a key bias)."""
    rows = np.zeros((B, Sq), bool)
    keys = np.zeros((B, Skv), bool)
    for b in range(B):
        A = allowed(kind, Sq, Skv, shift, None if kv_valid is None else kv_valid[b], window=window)
        if bias is not None:
            A = A & np.isfinite(np.asarray(bias[b]))[None, :]
        rows[b] = A.any(1)
        keys[b] = A.any(0)
    return rows, keys


def compare(got, ref, dtype, kind, shift=0, kv_valid=None, label="", zero_ref=(), window=None, frozen=0,
            bias=None, lse_rel=0.0):
    """Assert the tolerance bar; returns the error summary dict.

    ``zero_ref`` names tensors whose exact value is identically zero (e.g.
    dQ and dK when each query sees a single key): those are checked against
    an absolute bound instead of the relative one.
    """
    B, Hq, Sq, D = ref["O"].shape
    Skv = ref["dK"].shape[2]
    # ``lse_rel``: an extra LSE allowance relative to |LSE| (a few float32
    # ulps when LSE itself is large, e.g. under a large key-bias offset)
    rows, keys = structure(kind, B, Sq, Skv, shift, kv_valid, window, bias)
    keys[:, :frozen] = False      # frozen keys: dK = dV = 0 exactly
    errs = {}
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        g, r = got[name], ref[name]
        assert np.isfinite(g).all(), f"{label} {name}: non-finite values"
        if name in ("dK", "dV"):
            sel = np.broadcast_to(keys[:, None, :], g.shape[:3])
        else:
            sel = np.broadcast_to(rows[:, None, :], g.shape[:3])
        if name != "LSE":
            sel = sel[..., None]
        sel = np.broadcast_to(sel, g.shape)
        # exact zeros where nothing is attended
        dead = ~sel
        if dead.any():
            assert np.all(g[dead] == 0.0), f"{label} {name}: non-zero value where nothing is attended"
        if not sel.any():
            continue
        diff = np.abs(g - r)[sel]
        if dtype == "f32":
            errs[name] = float(diff.max())
            tol = TOL_F32 + (lse_rel * float(np.abs(r[sel]).max()) if name == "LSE" else 0.0)
            assert errs[name] <= tol, f"{label} {name}: max abs err {errs[name]:.3e}"
        elif name == "LSE":
            errs[name] = float(diff.max())
            tol = TOL_LSE_BF16 + lse_rel * float(np.abs(r[sel]).max())
            assert errs[name] <= tol, f"{label} LSE: max abs err {errs[name]:.3e}"
        elif name in zero_ref:
            assert float(np.abs(r[sel]).max()) < 1e-12, f"{label} {name}: reference not zero"
            errs[name] = float(diff.max())
            assert errs[name] <= 1e-3, f"{label} {name}: abs err {errs[name]:.3e} vs a zero reference"
        else:
            scale = float(np.abs(r[sel]).max())
            assert scale > 0, f"{label} {name}: reference is all zero (vacuous)"
            errs[name] = float(diff.max()) / scale
            assert errs[name] <= TOL_BF16[name], f"{label} {name}: rel err {errs[name]:.3e}"
    return errs


def check_case(q, k, v, do, kind, dtype, shift=0, kv_valid=None, scale=None, label="",
               zero_ref=(), ref_inputs=None, window=None, frozen=0, bias=None, lse_rel=0.0):
    say(f"[parity] {label} q{tuple(q.shape)} k{tuple(k.shape)} kind={kind} shift={shift} "
        f"kv_valid={kv_valid} window={window} frozen={frozen} bias={bias is not None} dtype={dtype}")
    got = run_gpu(q, k, v, do, kind, shift, kv_valid, scale, window=window, frozen=frozen, bias=bias)
    ref_in = (q, k, v, do) if ref_inputs is None else ref_inputs
    bias_np = None if bias is None else bias.detach().cpu().double().numpy()
    ref = attention_ref(*(x.double().numpy() for x in ref_in), kind, shift, kv_valid, scale,
                        window=window, bias=bias_np)
    errs = compare(got, ref, dtype, kind, shift, kv_valid, label, zero_ref, window, frozen, bias_np, lse_rel)
    say(f"[parity] {label} ok {errs}")
    return errs
