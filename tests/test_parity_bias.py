"""GPU parity of the per-batch key bias (fa_mask_desc.key_bias): bias[b, j]
added to the scaled score of every query row and head of batch entry b with
key j (the ggml playbook's additive mask, "3. Per-trainer porting
checklist", in its [B, Skv] form), against the fp64 oracle on the same
inputs, with parity_util's tolerances.  Biases are uniform in [-3, 3) with
about 15 % of the keys at -inf (those keys must get exactly dK = dV = 0).
"""
import numpy as np
import pytest
import torch

import flash_attention_fa_amd as fa
import workloads as W
from parity_util import check_case, run_gpu, say, to_np
from oracle import attention_ref

pytestmark = pytest.mark.gpu

FULL, CAUSAL, TTT, WINDOW = W.FULL, W.CAUSAL, W.TTT, W.WINDOW


def rand(shape, g, dtype):
    return torch.randn(*shape, generator=g).to(dtype)


def inputs(B, Hq, Hkv, Sq, Skv, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return (rand((B, Hq, Sq, D), g, dtype), rand((B, Hkv, Skv, D), g, dtype),
            rand((B, Hkv, Skv, D), g, dtype), rand((B, Hq, Sq, D), g, dtype))


CASES = [
    # label, B, Hq, Hkv, Sq, Skv, D, kind, shift, kv_valid, window
    ("full_sq_ne_skv", 2, 4, 2, 200, 333, 64, FULL, 0, None, None),
    ("causal_gqa_d128", 1, 8, 2, 320, 320, 128, CAUSAL, 0, None, None),
    ("causal_kvvalid_shift", 3, 4, 4, 257, 257, 64, CAUSAL, 3, (257, 100, 31), None),
    ("causal_prefix_d32", 2, 4, 2, 192, 256, 32, CAUSAL, -64, None, None),
    ("ttt_step2_d64", 2, 4, 2, 128, 384, 64, TTT, 0, (128, 77), None),
    ("ttt_step1_d128", 1, 8, 4, 192, 384, 128, TTT, 2, None, None),
    ("window_d32", 2, 4, 2, 300, 300, 32, WINDOW, 0, None, (48, 16)),
    ("causal_d16", 2, 4, 2, 260, 260, 16, CAUSAL, 0, None, None),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bias_parity(case, dtype):
    label, B, Hq, Hkv, Sq, Skv, D, kind, shift, kvv, win = case
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, do = inputs(B, Hq, Hkv, Sq, Skv, D, tdt, seed=hash(label) % 1000)
    bias = W.make_key_bias(B, Skv, seed=7)
    check_case(q, k, v, do, kind, dtype, shift, kvv, label=f"bias {label}", window=win, bias=bias)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bias_broadcast_row_and_empty_batch(dtype):
    # one bias row shared by every batch entry (stride 0), and a batch entry
    # whose keys are all -inf (every row empty: O = LSE = dQ = 0, dK = dV = 0)
    B, Hq, Hkv, S, D = 3, 4, 2, 200, 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, do = inputs(B, Hq, Hkv, S, S, D, tdt, seed=21)
    row = W.make_key_bias(1, S, seed=3)
    check_case(q, k, v, do, CAUSAL, dtype, label="bias broadcast", bias=row.expand(B, S))
    bias = W.make_key_bias(B, S, seed=4)
    bias[1] = float("-inf")
    check_case(q, k, v, do, CAUSAL, dtype, label="bias empty batch", bias=bias)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bias_large_common_offset(dtype):
    # a bias with a large common part (far beyond the running max's slack of
    # 8 in log2 units): softmax keeps only the differences, LSE carries the
    # offset.  The scores are formed in float32, so each carries about
    # |offset| * 2^-24 of rounding, which every output inherits as a relative
    # error: the float32 bar (1e-4 absolute, made for moderate scores) takes
    # offsets of 100 and 200, bfloat16's relative bar 1000 and 2000.  LSE is
    # itself a float32 near the offset: it gets an allowance of four ulps,
    # 2^-21 |LSE|, on top of the usual bound.
    B, Hq, Hkv, S, D = 2, 4, 2, 256, 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, do = inputs(B, Hq, Hkv, S, S, D, tdt, seed=22)
    off = torch.tensor([[1000.0], [-2000.0]]) if dtype == "bf16" else torch.tensor([[100.0], [-200.0]])
    bias = W.make_key_bias(B, S, seed=5, neg_inf_frac=0.0) + off
    check_case(q, k, v, do, FULL, dtype, label="bias offset", bias=bias, lse_rel=2.0 ** -21)


MANY = [
    # enough query rows for the one-launch backward (dK/dV and dQ together)
    ("split_causal", 1, 32, 4, 2048, 2048, 128, CAUSAL, None),
    ("unsplit_full_d64", 4, 32, 32, 512, 512, 64, FULL, None),
    ("ttt_many", 1, 32, 8, 1024, 2048, 64, TTT, None),
]


@pytest.mark.parametrize("case", MANY, ids=[c[0] for c in MANY])
def test_bias_many_workgroups_staged_equals_fused(case):
    # the whole backward (one launch for dK/dV and dQ where shapes allow)
    # against the stages run one by one: bitwise; and the result against the
    # oracle on a sample of heads
    label, B, Hq, Hkv, Sq, Skv, D, kind, kvv = case
    say(f"[bias] many workgroups {label}")
    q, k, v, do = (x.cuda() for x in inputs(B, Hq, Hkv, Sq, Skv, D, torch.bfloat16, seed=31))
    bias = W.make_key_bias(B, Skv, seed=8, device="cuda")
    o, lse = fa.fa_fwd(q, k, v, mask_kind=kind, key_bias=bias)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, mask_kind=kind, key_bias=bias)
    sq, sk, sv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(q, k, mask_kind=kind, key_bias=bias), dtype=torch.uint8,
                     device="cuda")
    for st in (fa.FA_BWD_DELTA, fa.FA_BWD_DKDV, fa.FA_BWD_DQ):
        fa.fa_bwd_stage(st, q, k, v, o, lse, do, sq, sk, sv, ws, mask_kind=kind, key_bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(dq, sq) and torch.equal(dk, sk) and torch.equal(dv, sv)
    # rerun: bitwise the same
    dq2, dk2, dv2 = fa.fa_bwd(q, k, v, o, lse, do, mask_kind=kind, key_bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    # O and LSE of two heads against the oracle
    G = Hq // Hkv
    heads = [0, Hq - 1]
    ref = attention_ref(*(x.cpu().double().numpy() for x in (q, k, v, do)), kind,
                        heads=heads, bias=bias.cpu().double().numpy())
    for h in heads:
        o_err = np.abs(to_np(o[:, h]) - ref["O"][:, h]).max() / np.abs(ref["O"][:, h]).max()
        l_err = np.abs(to_np(lse[:, h]) - ref["LSE"][:, h]).max()
        dq_err = np.abs(to_np(dq[:, h]) - ref["dQ"][:, h]).max() / np.abs(ref["dQ"][:, h]).max()
        say(f"[bias] {label} head {h}: O {o_err:.2e} LSE {l_err:.2e} dQ {dq_err:.2e}")
        assert o_err <= 2e-2 and l_err <= 1e-2 and dq_err <= 5e-2
    del G


def test_bias_noalloc_equals_fa_fwd():
    B, Hq, Hkv, S, D = 2, 8, 2, 384, 128
    q, k, v, _ = (x.cuda() for x in inputs(B, Hq, Hkv, S, S, D, torch.bfloat16, seed=41))
    bias = W.make_key_bias(B, S, seed=9, device="cuda")
    o1, l1 = fa.fa_fwd(q, k, v, mask_kind=CAUSAL, key_bias=bias)
    o2, l2 = fa.fa_fwd_noalloc(q, k, v, mask_kind=CAUSAL, key_bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bias_autograd():
    B, Hq, Hkv, S, D = 2, 4, 2, 160, 64
    q, k, v, do = inputs(B, Hq, Hkv, S, S, D, torch.float32, seed=51)
    bias = W.make_key_bias(B, S, seed=10)
    leaves = [x.cuda().requires_grad_(True) for x in (q, k, v)]
    out = fa.attention(*leaves, mask_kind=CAUSAL, key_bias=bias.cuda())
    out.backward(do.cuda())
    torch.cuda.synchronize()
    ref = attention_ref(*(x.double().numpy() for x in (q, k, v, do)), CAUSAL,
                        bias=bias.double().numpy())
    assert np.abs(to_np(out) - ref["O"]).max() <= 1e-4
    for t, name in zip(leaves, ("dQ", "dK", "dV")):
        assert np.abs(to_np(t.grad) - ref[name]).max() <= 1e-4, name


def test_no_bias_results_unchanged_by_a_zero_bias():
    # a zero bias goes through the bias kernels; results equal the no-bias
    # kernels' to rounding (the scores start from +0 instead of 0)
    B, Hq, Hkv, S, D = 1, 8, 2, 320, 128
    q, k, v, do = inputs(B, Hq, Hkv, S, S, D, torch.bfloat16, seed=61)
    a = run_gpu(q, k, v, do, CAUSAL)
    z = run_gpu(q, k, v, do, CAUSAL, bias=torch.zeros(B, S))
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[name], z[name]), name
