"""fa_fwd_noalloc (the forward whose workspace is the library's static
device array, for callers that cannot allocate) against fa_fwd, through the
C ABI: two calls in a row, the second on a smaller input (so the array holds
the first call's larger V^T when the second runs), each bitwise equal to
fa_fwd on the same inputs, the first also within the bf16 bars of the fp64
oracle; a shape beyond the array is refused before any launch."""
import numpy as np
import pytest
import torch

import flash_attention_fa_amd as fa
import workloads as W
from flash_attention_fa_amd import _lib
from oracle import attention_ref
from parity_util import TOL_BF16, TOL_LSE_BF16, say

pytestmark = pytest.mark.gpu


def inputs(B, Hq, Hkv, Sq, Skv, D, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    mk = lambda H, S: torch.randn(B, H, S, D, generator=g).to(torch.bfloat16)
    return mk(Hq, Sq), mk(Hkv, Skv), mk(Hkv, Skv)


CALLS = [
    # B, Hq, Hkv, Sq, Skv, D, kind, kv_valid
    (2, 8, 2, 1000, 1000, 128, W.CAUSAL, None),
    (1, 4, 2, 333, 333, 64, W.FULL, (200,)),
]


def test_noalloc_matches_fa_fwd_on_two_calls():
    for n, (B, Hq, Hkv, Sq, Skv, D, kind, kvv) in enumerate(CALLS):
        say(f"[noalloc] call {n}: B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} D={D} kind={kind} kv_valid={kvv}")
        q, k, v = inputs(B, Hq, Hkv, Sq, Skv, D, seed=700 + n)
        qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
        kv = None if kvv is None else torch.tensor(kvv, dtype=torch.int32, device="cuda")
        kw = dict(mask_kind=kind, kv_valid=kv)
        o_ref, lse_ref = fa.fa_fwd(qg, kg, vg, **kw)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(lse_ref, float("nan"))
        fa.fa_fwd_noalloc(qg, kg, vg, out=o, lse=lse, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"call {n}: O differs from fa_fwd"
        assert torch.equal(lse, lse_ref), f"call {n}: LSE differs from fa_fwd"
        if n == 0:
            ref = attention_ref(*(x.double().numpy() for x in (q, k, v, q)), kind, 0, kvv)
            O, L = o.float().cpu().numpy(), lse.cpu().numpy()
            err_o = np.abs(O - ref["O"]).max() / np.abs(ref["O"]).max()
            err_l = np.abs(L - ref["LSE"]).max()
            assert err_o <= TOL_BF16["O"] and err_l <= TOL_LSE_BF16, (err_o, err_l)
        say(f"[noalloc] call {n} ok")


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    # Skv such that V^T needs more than the static array (nothing launched)
    B, Hq, Hkv, D = 1, 8, 4, 128
    Skv = _lib.FWD_NOALLOC_SCRATCH_BYTES // (2 * B * Hkv * D) + 64
    q = torch.zeros(B, Hq, 64, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, Hkv, Skv, D, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_noalloc(q, k, k.clone(), mask_kind=W.FULL)
    assert e.value.status == _lib.FA_ERR_UNSUPPORTED and "scratch" in str(e.value)
