"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes that the oracle finishes in seconds but that still span several
tiles and a ragged tail, for every mask kind, GQA ratio, head dim, dtype,
padding and stride layout; plus the edge cases (single row/key, empty key set,
NaN in padded rows, fully-masked rows) and bitwise determinism.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity_util import check_case, run_gpu, say

pytestmark = pytest.mark.gpu

FULL, CAUSAL, TTT, WINDOW = W.FULL, W.CAUSAL, W.TTT, W.WINDOW


def rnd(shape, seed, dtype):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def inputs(B, Hq, Hkv, Sq, Skv, D, dtype, seed=0):
    return (rnd((B, Hq, Sq, D), seed, dtype), rnd((B, Hkv, Skv, D), seed + 1, dtype),
            rnd((B, Hkv, Skv, D), seed + 2, dtype), rnd((B, Hq, Sq, D), seed + 3, dtype))


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", [CAUSAL, FULL])
def test_bf16_self_attention_ragged(D, kind):
    q, k, v, do = inputs(2, 4, 2, 300, 300, D, torch.bfloat16, seed=D)
    check_case(q, k, v, do, kind, "bf16", label=f"bf16 self D={D}")


@pytest.mark.parametrize("G", [1, 8])
def test_bf16_gqa_causal(G):
    q, k, v, do = inputs(1, 8, 8 // G, 520, 520, 128, torch.bfloat16, seed=7)
    check_case(q, k, v, do, CAUSAL, "bf16", label=f"bf16 gqa G={G}")


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("G", [2, 3])
def test_bf16_gqa_group_split(G, D):
    # The dK/dV kernel splits each key block's work between two workgroups: by
    # halves of the group's heads when G is even, by halves of the steps when odd
    q, k, v, do = inputs(2, 2 * G, 2, 300, 300, D, torch.bfloat16, seed=13 + G + D)
    check_case(q, k, v, do, CAUSAL, "bf16", label=f"bf16 gqa split G={G} D={D}")


def test_bf16_cross_attention_padded_keys():
    # Sq != Skv, per-batch valid key counts that are not tile multiples
    q, k, v, do = inputs(2, 4, 4, 200, 333, 64, torch.bfloat16, seed=11)
    check_case(q, k, v, do, FULL, "bf16", kv_valid=(300, 77), label="bf16 cross kv_valid")


def test_bf16_padded_rows_hold_nan():
    # NaN in K/V rows past kv_valid must never reach the outputs.
    q, k, v, do = inputs(2, 2, 2, 130, 200, 64, torch.bfloat16, seed=13)
    kv_valid = (150, 61)
    clean = run_gpu(q, k, v, do, FULL, 0, kv_valid)
    k2, v2 = k.clone(), v.clone()
    for b, n in enumerate(kv_valid):
        k2[b, :, n:] = float("nan")
        v2[b, :, n:] = float("nan")
    dirty = run_gpu(q, k2, v2, do, FULL, 0, kv_valid)
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(clean[name], dirty[name]), name
    # the oracle's own P.V would propagate the NaN (0 * NaN), so it sees the
    # clean values; the GPU sees the NaN-filled ones
    check_case(q, k2, v2, do, FULL, "bf16", kv_valid=kv_valid, label="bf16 nan padding",
               ref_inputs=(q, k, v, do))


@pytest.mark.parametrize("shift", [1, 3, 70])
def test_bf16_causal_shift_with_empty_rows(shift):
    q, k, v, do = inputs(1, 2, 1, 257, 257, 64, torch.bfloat16, seed=17)
    check_case(q, k, v, do, CAUSAL, "bf16", shift=shift, label=f"bf16 causal shift={shift}")


def test_bf16_causal_sq_ne_skv():
    q, k, v, do = inputs(1, 4, 2, 150, 400, 64, torch.bfloat16, seed=19)
    check_case(q, k, v, do, CAUSAL, "bf16", label="bf16 causal Sq<Skv")
    q, k, v, do = inputs(1, 4, 2, 400, 150, 64, torch.bfloat16, seed=20)
    check_case(q, k, v, do, CAUSAL, "bf16", label="bf16 causal Sq>Skv")


@pytest.mark.parametrize("L,t,shift,kvv", [
    (256, 2, 0, None), (130, 1, 0, None), (130, 2, 2, None), (100, 2, 0, (70,)),
    (300, 0, 0, None), (96, 3, 1, (90,)),
    # short steps: the ragged last key tile reaches past Skv into positions
    # that the rows of one 32-row block would match
    (40, 1, 0, None), (20, 2, 0, None), (50, 3, 1, (45,))])
def test_bf16_ttt(L, t, shift, kvv):
    q, k, v, do = inputs(1, 8, 2, L, (t + 1) * L, 128, torch.bfloat16, seed=L + t)
    check_case(q, k, v, do, TTT, "bf16", shift=shift, kv_valid=kvv,
               label=f"bf16 ttt L={L} t={t} shift={shift}")


@pytest.mark.parametrize("D", [16, 32, 64])
def test_bf16_ttt_small_head_dim(D):
    q, k, v, do = inputs(1, 4, 2, 130, 390, D, torch.bfloat16, seed=D + 5)
    check_case(q, k, v, do, TTT, "bf16", kv_valid=(100,), label=f"bf16 ttt D={D}")


# WINDOW: (left, right) bands, with shift, padding, GQA, Sq != Skv, and
# bands narrower than a 64-key tile, wider than several, and one-sided.
WIN_CASES = [
    # B, Hq, Hkv, Sq, Skv, shift, kv_valid, (left, right)
    (2, 4, 2, 300, 300, 0, None, (63, 0)),
    (2, 4, 4, 300, 300, 0, None, (40, 40)),
    (1, 8, 2, 333, 333, 3, (290,), (100, 7)),
    (2, 2, 1, 200, 333, 0, (333, 120), (5, 150)),
    (1, 4, 2, 260, 260, 70, None, (0, 0)),
]


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("case", WIN_CASES, ids=[f"w{c[7][0]}_{c[7][1]}_s{c[5]}" for c in WIN_CASES])
def test_bf16_window(case, D):
    B, Hq, Hkv, Sq, Skv, shift, kvv, win = case
    q, k, v, do = inputs(B, Hq, Hkv, Sq, Skv, D, torch.bfloat16, seed=D + Sq + win[0])
    # a band of one key: P = 1 and dS = 0 on every row, so dQ and dK are exactly 0
    zero = ("dQ", "dK") if win == (0, 0) else ()
    check_case(q, k, v, do, WINDOW, "bf16", shift=shift, kv_valid=kvv, window=win,
               label=f"bf16 window {win} shift={shift} D={D}", zero_ref=zero)


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_window_many_workgroups(D):
    q, k, v, do = inputs(4, 128, 16, 300, 333, D, torch.bfloat16, seed=81 + D)
    check_case(q, k, v, do, WINDOW, "bf16", shift=1, kv_valid=(333, 300, 77, 1), window=(90, 30),
               label=f"bf16 many-WG window D={D}")


def test_f32_window():
    q, k, v, do = inputs(1, 4, 2, 150, 150, 64, torch.float32, seed=91)
    check_case(q, k, v, do, WINDOW, "f32", shift=2, kv_valid=(140,), window=(20, 9),
               label="f32 window")


def test_bf16_bshd_strided_views():
    # q/k/v/dO as transposed views of [B, S, H, D] storage (no copies)
    B, S, Hq, Hkv, D = 2, 190, 4, 2, 64
    g = torch.Generator("cpu").manual_seed(23)
    mk = lambda H: torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).transpose(1, 2)
    q, k, v, do = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    assert not q.is_contiguous()
    check_case(q, k, v, do, CAUSAL, "bf16", label="bf16 bshd views")


def test_bf16_explicit_scale():
    q, k, v, do = inputs(1, 2, 2, 128, 128, 64, torch.bfloat16, seed=29)
    check_case(q, k, v, do, CAUSAL, "bf16", scale=0.05, label="bf16 scale=0.05")


def test_bf16_single_row_and_key():
    # one key per row: the softmax is constant, so dQ and dK are exactly zero
    q, k, v, do = inputs(1, 1, 1, 1, 1, 32, torch.bfloat16, seed=31)
    check_case(q, k, v, do, CAUSAL, "bf16", label="bf16 1x1", zero_ref=("dQ", "dK"))


def test_bf16_no_valid_keys():
    q, k, v, do = inputs(2, 2, 2, 64, 64, 64, torch.bfloat16, seed=37)
    got = run_gpu(q, k, v, do, FULL, 0, (0, 0))
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.all(got[name] == 0.0), name


@pytest.mark.parametrize("kind", [CAUSAL, FULL])
def test_f32_tiny(kind):
    w = W.tiny_fp32(kind)
    q, k, v, do = W.make_inputs(w, seed=0)
    check_case(q, k, v, do, kind, "f32", label=f"{w.name}")


@pytest.mark.parametrize("D", [16, 128])
def test_f32_ragged_gqa_ttt(D):
    q, k, v, do = inputs(1, 4, 2, 70, 210, D, torch.float32, seed=41)
    check_case(q, k, v, do, TTT, "f32", kv_valid=(65,), label=f"f32 ttt D={D}")
    q, k, v, do = inputs(2, 4, 1, 99, 99, D, torch.float32, seed=43)
    check_case(q, k, v, do, CAUSAL, "f32", shift=2, label=f"f32 causal D={D}")


@pytest.mark.parametrize("kind", [CAUSAL, TTT, WINDOW])
def test_bitwise_determinism(kind):
    L = 384
    Skv = 3 * L if kind == TTT else L
    q, k, v, do = inputs(1, 8, 2, L, Skv, 128, torch.bfloat16, seed=47)
    win = (100, 20) if kind == WINDOW else None
    say(f"[determinism] kind={kind}")
    a = run_gpu(q, k, v, do, kind, window=win)
    # unrelated work in between, then the same call again
    x = torch.randn(4096, 4096, device="cuda")
    (x @ x).sum().item()
    b = run_gpu(q, k, v, do, kind, window=win)
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[name], b[name]), name


STAGED = [
    # dtype, D, B, Hq, Hkv, L, kind
    (torch.bfloat16, 16, 1, 8, 2, 320, CAUSAL), (torch.bfloat16, 64, 1, 8, 2, 320, CAUSAL),
    (torch.bfloat16, 128, 1, 8, 2, 320, CAUSAL), (torch.float32, 64, 1, 8, 2, 320, CAUSAL),
    # 512+ dQ workgroups of 256 rows: fa_bwd runs dK/dV and dQ as one launch
    (torch.bfloat16, 128, 4, 128, 16, 300, CAUSAL), (torch.bfloat16, 64, 4, 128, 16, 300, TTT),
    (torch.bfloat16, 32, 4, 128, 16, 300, WINDOW), (torch.bfloat16, 64, 16, 64, 64, 256, CAUSAL),
]


@pytest.mark.parametrize("case", STAGED, ids=[f"{str(c[0])[6:]}_D{c[1]}_B{c[2]}_H{c[3]}_{W.KIND_NAMES[c[6]]}"
                                               for c in STAGED])
def test_staged_backward_equals_fa_bwd(case):
    """fa_bwd_stage DELTA, DKDV, DQ in turn writes bitwise what fa_bwd writes
    (the dK/dV stage is the split kernel and its reduction; with
    enough query rows fa_bwd launches the dK/dV and dQ workgroups together)."""
    import flash_attention_fa_amd as fa
    dtype, D, B, Hq, Hkv, L, kind = case
    Skv = 3 * L if kind == TTT else L
    win = (50, 7) if kind == WINDOW else None
    q, k, v, do = (x.cuda() for x in inputs(B, Hq, Hkv, L, Skv, D, dtype, seed=53))
    say(f"[staged] {case}")
    kw = dict(mask_kind=kind, window=win)
    o, lse = fa.fa_fwd(q, k, v, **kw)
    ref = fa.fa_bwd(q, k, v, o, lse, do, **kw)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(q, k, mask_kind=kind), dtype=torch.uint8, device="cuda")
    # the gradient stages in the opposite order: they are independent once Delta exists
    for stage in (fa.FA_BWD_DELTA, fa.FA_BWD_DQ, fa.FA_BWD_DKDV):
        fa.fa_bwd_stage(stage, q, k, v, o, lse, do, dq, dk, dv, ws, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), ref, (dq, dk, dv)):
        assert torch.equal(a, b), name


# Launches with at least 512 workgroups of 256 query rows (B*Hq*ceil(Sq/256))
# take the 8-wave forward and dQ kernels (256 query rows per workgroup); these
# cases reach them with ragged tiles, GQA, every mask kind and padding.
MANY = [
    ("causal", CAUSAL, 300, 300, 0, None),
    ("full_kv_valid", FULL, 300, 333, 0, (333, 300, 77, 1)),
    ("ttt_t2", TTT, 300, 900, 0, (300, 250, 1, 299)),
    ("causal_shift5", CAUSAL, 300, 300, 5, None),
    # short TTT steps: a ragged last key tile reaching past Skv
    ("ttt_short", TTT, 40, 120, 0, (40, 33, 1, 40)),
]


@pytest.mark.parametrize("case", MANY, ids=[c[0] for c in MANY])
def test_bf16_many_workgroups(case):
    name, kind, Sq, Skv, shift, kvv = case
    q, k, v, do = inputs(4, 128, 16, Sq, Skv, 128, torch.bfloat16, seed=61)
    check_case(q, k, v, do, kind, "bf16", shift=shift, kv_valid=kvv, label=f"bf16 many-WG {name}")


@pytest.mark.parametrize("D", [16, 32, 64])
@pytest.mark.parametrize("case", MANY[:3], ids=[c[0] for c in MANY[:3]])
def test_bf16_many_workgroups_small_head_dim(case, D):
    name, kind, Sq, Skv, shift, kvv = case
    q, k, v, do = inputs(4, 128, 16, Sq, Skv, D, torch.bfloat16, seed=71 + D)
    check_case(q, k, v, do, kind, "bf16", shift=shift, kv_valid=kvv, label=f"bf16 many-WG {name} D={D}")


# At least 1024 key blocks of 256 (B * Hkv * ceil(keys / 256)): the
# dK/dV kernel then gives each block to one workgroup, which writes dK and dV
# itself (no partial sums, no reduction).
UNSPLIT = [
    # name, B, Hq, Hkv, Sq, Skv, D, kind, shift, kv_valid, window
    ("mha_causal_d128", 16, 64, 64, 256, 256, 128, CAUSAL, 0, None, None),
    ("gqa_full_kvvalid_d128", 8, 256, 128, 200, 256, 128, FULL, 0, (256, 255, 130, 1, 64, 200, 7, 99), None),
    ("ttt_d64", 8, 256, 128, 256, 512, 64, TTT, 0, None, None),
    ("window_d32", 16, 64, 64, 256, 256, 32, WINDOW, 2, None, (30, 10)),
    ("causal_kvvalid_d16", 16, 64, 64, 256, 256, 16, CAUSAL, 1, (256, 255, 130, 1, 64, 200, 7, 99) * 2, None),
    ("ttt_d16", 8, 256, 128, 256, 512, 16, TTT, 0, None, None),
]


@pytest.mark.parametrize("case", UNSPLIT, ids=[c[0] for c in UNSPLIT])
def test_bf16_dkdv_unsplit(case):
    name, B, Hq, Hkv, Sq, Skv, D, kind, shift, kvv, win = case
    q, k, v, do = inputs(B, Hq, Hkv, Sq, Skv, D, torch.bfloat16, seed=101 + D)
    check_case(q, k, v, do, kind, "bf16", shift=shift, kv_valid=kvv, window=win, label=f"bf16 unsplit {name}")


def test_bf16_many_workgroups_nan_padding():
    q, k, v, do = inputs(4, 128, 16, 300, 333, 128, torch.bfloat16, seed=67)
    kv_valid = (333, 300, 77, 1)
    say("[many-WG nan padding]")
    clean = run_gpu(q, k, v, do, FULL, 0, kv_valid)
    k2, v2 = k.clone(), v.clone()
    for b, n in enumerate(kv_valid):
        k2[b, :, n:] = float("nan")
        v2[b, :, n:] = float("nan")
    dirty = run_gpu(q, k2, v2, do, FULL, 0, kv_valid)
    for nm in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(clean[nm], dirty[nm]), nm


# Prefix: CAUSAL with a negative shift -P over Skv = P + Sq keys (every query
# sees the P prefix keys, then the causal part), with and without the prefix
# frozen (its dK, dV exactly 0, the rest unchanged).
PREFIX = [
    # name, B, Hq, Hkv, Sq, P, frozen
    ("p37", 2, 4, 2, 200, 37, 0),
    ("p37_frozen", 2, 4, 2, 200, 37, 37),
    ("p256_frozen", 1, 8, 2, 300, 256, 256),
    ("p300_frozen_part", 2, 4, 4, 130, 300, 170),   # frozen part of the prefix only
]


@pytest.mark.parametrize("D", [16, 64, 128])
@pytest.mark.parametrize("case", PREFIX, ids=[c[0] for c in PREFIX])
def test_bf16_prefix(case, D):
    name, B, Hq, Hkv, Sq, P, frozen = case
    q, k, v, do = inputs(B, Hq, Hkv, Sq, P + Sq, D, torch.bfloat16, seed=131 + D)
    check_case(q, k, v, do, CAUSAL, "bf16", shift=-P, frozen=frozen, label=f"bf16 prefix {name} D={D}")


def test_bf16_prefix_window_and_f32():
    q, k, v, do = inputs(2, 4, 2, 150, 190, 64, torch.bfloat16, seed=141)
    check_case(q, k, v, do, WINDOW, "bf16", shift=-40, window=(60, 10), frozen=20, label="bf16 window shift=-40")
    q, k, v, do = inputs(1, 2, 1, 100, 164, 64, torch.float32, seed=142)
    check_case(q, k, v, do, CAUSAL, "f32", shift=-64, frozen=64, label="f32 prefix P=64 frozen")


def test_bf16_prefix_many_workgroups_and_ttt_frozen():
    # 512+ forward workgroups, the split dK/dV kernel with frozen blocks
    q, k, v, do = inputs(4, 128, 16, 300, 556, 128, torch.bfloat16, seed=151)
    check_case(q, k, v, do, CAUSAL, "bf16", shift=-256, frozen=256, label="bf16 many-WG prefix 256 frozen")
    # TTT keys of later steps below frozen_keys are frozen too
    q, k, v, do = inputs(1, 4, 2, 100, 300, 128, torch.bfloat16, seed=152)
    check_case(q, k, v, do, TTT, "bf16", frozen=150, label="bf16 ttt frozen 150")


def test_bf16_prefix_unsplit_frozen():
    # 1024+ key blocks: the unsplit dK/dV kernel writes frozen keys itself
    q, k, v, do = inputs(16, 64, 64, 128, 384, 64, torch.bfloat16, seed=161)
    check_case(q, k, v, do, CAUSAL, "bf16", shift=-256, frozen=200, label="bf16 unsplit prefix frozen 200")
