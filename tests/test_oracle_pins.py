"""Pins for the fp64 oracle against things other than itself.

Each test ties a part of ``oracle/`` to the mathematics or to an independent
library routine, chosen so that a plausible slip (a dropped term, a wrong sign
or index, a transposed operand, a wrong mask index) fails at least one:

* closed forms derived by hand (tests/golden/closed_forms.json);
* torch's fp64 ``scaled_dot_product_attention`` and its autograd (the
  reference arm of the CS336 benchmark), including its GQA convention;
* ``torch.logsumexp`` on library-built masked scores for LSE;
* central finite differences of L = sum(O * dO) for every mask kind;
* invariants (rows of P sum to 1, equal keys, causal row 0, key shift,
  sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, Delta = rowsum(dO * O));
* the step-by-step EAGLE3 TTT formulation (oracle/ttt_steps.py);
* brute force of the SpecForge mask functions, pair by pair;
* padding equals truncation; padded keys get exactly-zero gradients;
* WINDOW: torch fp64 SDPA and autograd with a band mask built by
  torch.tril / torch.triu, the limits that reduce it to CAUSAL and FULL,
  finite differences, the gradient invariants, and pair counts in closed form.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (FULL, CAUSAL, TTT, WINDOW, allowed, attention_forward,
                    attention_backward, attention_ref, allowed_pair_count,
                    ttt_stepwise_forward)

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(shape, seed, lo=None):
    g = np.random.default_rng(seed)
    if lo is None:
        return g.standard_normal(shape)
    return g.uniform(lo, -lo, shape)


# --------------------------------------------------------------------------
# closed forms

def _ev(x):
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, {"ln": math.log}))


def _arr(rows):
    return np.array([[_ev(x) for x in r] for r in rows])


@pytest.mark.parametrize("case", json.load(open(os.path.join(
    HERE, "golden", "closed_forms.json")))["cases"], ids=lambda c: c["name"])
def test_closed_forms(case):
    q = _arr(case["q"])[None, None]
    k = _arr(case["k"])[None, None]
    v = _arr(case["v"])[None, None]
    do = _arr(case["do"])[None, None]
    r = attention_ref(q, k, v, do, case["kind"], case["shift"], None,
                      case["scale"])
    np.testing.assert_allclose(r["O"][0, 0], _arr(case["O"]), atol=1e-14)
    np.testing.assert_allclose(r["LSE"][0, 0], [_ev(x) for x in case["LSE"]],
                               atol=1e-14)
    for name in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(r[name][0, 0], _arr(case[name]), atol=1e-14,
                                   err_msg=name)


# --------------------------------------------------------------------------
# library routines: torch fp64 SDPA, logsumexp, autograd

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (8, 1)])
@pytest.mark.parametrize("S,D", [(7, 4), (33, 16), (64, 8)])
def test_forward_and_grads_match_torch_sdpa(causal, Hq, Hkv, S, D):
    B = 2
    q = _rand((B, Hq, S, D), 1)
    k = _rand((B, Hkv, S, D), 2)
    v = _rand((B, Hkv, S, D), 3)
    do = _rand((B, Hq, S, D), 4)
    kind = CAUSAL if causal else FULL
    r = attention_ref(q, k, v, do, kind)

    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, enable_gqa=Hq != Hkv)
    out.backward(torch.tensor(do))
    np.testing.assert_allclose(r["O"], out.detach().numpy(), atol=1e-12)
    for name, t in (("dQ", tq), ("dK", tk), ("dV", tv)):
        ref = t.grad.numpy()
        assert np.abs(ref).max() > 1e-3          # non-vacuous gradient
        np.testing.assert_allclose(r[name], ref, atol=1e-11, err_msg=name)

    # LSE: torch.logsumexp over scores masked with torch.tril
    kk = torch.tensor(k).repeat_interleave(Hq // Hkv, dim=1)
    scores = torch.tensor(q) @ kk.transpose(-1, -2) / math.sqrt(D)
    if causal:
        keep = torch.ones(S, S, dtype=torch.bool).tril()
        scores = scores.masked_fill(~keep, -math.inf)
    np.testing.assert_allclose(r["LSE"], torch.logsumexp(scores, -1).numpy(),
                               atol=1e-12)


def test_explicit_scale_matches_sdpa():
    q, k, v = _rand((1, 2, 9, 8), 5), _rand((1, 2, 11, 8), 6), _rand((1, 2, 11, 8), 7)
    O, _ = attention_forward(q, k, v, FULL, scale=0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.tensor(x) for x in (q, k, v)), scale=0.3)
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12)


def test_sq_ne_skv_full_matches_sdpa():
    q, k, v = _rand((2, 3, 5, 8), 8), _rand((2, 3, 13, 8), 9), _rand((2, 3, 13, 8), 10)
    O, _ = attention_forward(q, k, v, FULL)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.tensor(x) for x in (q, k, v)))
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12)


# --------------------------------------------------------------------------
# finite differences (every mask kind, GQA, padding, shift)

FD_CASES = [
    # kind, B, Hq, Hkv, Sq, Skv, D, shift, kv_valid
    (FULL, 1, 2, 1, 5, 7, 4, 0, None),
    (FULL, 2, 2, 2, 6, 9, 4, 0, (9, 4)),
    (CAUSAL, 1, 4, 2, 8, 8, 4, 0, None),
    (CAUSAL, 1, 2, 2, 9, 9, 8, 2, (6,)),
    (CAUSAL, 1, 1, 1, 6, 10, 4, 0, None),
    (TTT, 1, 2, 1, 5, 15, 4, 0, None),
    (TTT, 1, 2, 2, 6, 12, 4, 1, (4,)),
    (TTT, 2, 4, 2, 4, 8, 8, 0, (4, 3)),
    # WINDOW (left, right)
    (WINDOW, 1, 2, 1, 9, 9, 4, 0, None, (2, 0)),
    (WINDOW, 2, 4, 2, 8, 11, 4, 1, (11, 6), (1, 3)),
]


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: f"k{c[0]}_{c[4]}x{c[5]}")
def test_backward_matches_finite_differences(case):
    kind, B, Hq, Hkv, Sq, Skv, D, shift, kvv = case[:9]
    win = case[9] if len(case) > 9 else None
    q = _rand((B, Hq, Sq, D), 11)
    k = _rand((B, Hkv, Skv, D), 12)
    v = _rand((B, Hkv, Skv, D), 13)
    do = _rand((B, Hq, Sq, D), 14)
    dQ, dK, dV, _ = attention_backward(q, k, v, do, kind, shift, kvv, window=win)

    def loss(q_, k_, v_):
        O, _ = attention_forward(q_, k_, v_, kind, shift, kvv, window=win)
        return float((O * do).sum())

    h = 1e-6
    for name, x, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        assert np.abs(grad).max() > 1e-3, name       # trap 7: non-zero gradient
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.abs(num - grad).max() / np.abs(grad).max()
        assert err < 1e-6, (name, err)


# --------------------------------------------------------------------------
# invariants

def test_rows_of_p_sum_to_one_and_equal_keys_are_uniform():
    B, H, S, D = 1, 2, 12, 8
    q = _rand((B, H, S, D), 20)
    k_row = _rand((D,), 21)
    k = np.broadcast_to(k_row, (B, H, S, D)).copy()
    v = _rand((B, H, S, D), 22)
    for kind in (FULL, CAUSAL):
        # V = ones -> O = 1 exactly when the rows of P sum to 1
        O1, _ = attention_forward(q, k, np.ones_like(v), kind)
        np.testing.assert_allclose(O1, 1.0, atol=1e-14)
        O, LSE = attention_forward(q, k, v, kind)
        n = np.arange(1, S + 1) if kind == CAUSAL else np.full(S, S)
        for i in range(S):
            mean = v[0, :, : n[i]].mean(axis=1)
            np.testing.assert_allclose(O[0, :, i], mean, atol=1e-13)
            expect = q[0, :, i] @ k_row / math.sqrt(D) + math.log(n[i])
            np.testing.assert_allclose(LSE[0, :, i], expect, atol=1e-13)


def test_causal_row_zero_and_key_shift():
    B, H, S, D = 1, 3, 10, 16
    q, k, v = _rand((B, H, S, D), 30), _rand((B, H, S, D), 31), _rand((B, H, S, D), 32)
    O, LSE = attention_forward(q, k, v, CAUSAL)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], atol=1e-14)
    np.testing.assert_allclose(LSE[:, :, 0],
                               (q[:, :, 0] * k[:, :, 0]).sum(-1) / 4.0, atol=1e-14)
    c = _rand((D,), 33)
    O2, LSE2 = attention_forward(q, k + c, v, CAUSAL)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(LSE2, LSE + (q @ c) / 4.0, atol=1e-12)


@pytest.mark.parametrize("kind,shift,kvv,win", [(FULL, 0, (7,), None), (CAUSAL, 3, None, None),
                                                (TTT, 0, (5,), None), (TTT, 2, None, None),
                                                (WINDOW, 2, (9,), (2, 1))])
def test_gradient_sum_invariants(kind, shift, kvv, win):
    B, Hq, Hkv, Sq, D = 1, 4, 2, 8, 8
    Skv = 3 * Sq if kind == TTT else 11
    q = _rand((B, Hq, Sq, D), 40)
    k, v = _rand((B, Hkv, Skv, D), 41), _rand((B, Hkv, Skv, D), 42)
    do = _rand((B, Hq, Sq, D), 43)
    r = attention_ref(q, k, v, do, kind, shift, kvv, window=win)
    # sum_j dS_ij = 0  =>  sum_j dK_j = 0 per (b, kv head)
    np.testing.assert_allclose(r["dK"].sum(axis=2), 0.0, atol=1e-12)
    # sum_j P_ij = 1  =>  sum_j dV_j = sum over non-empty rows of dO_i (per group)
    G = Hq // Hkv
    nonempty = allowed(kind, Sq, Skv, shift, None if kvv is None else kvv[0], window=win).any(1)
    expect = do[:, :, nonempty].sum(axis=2).reshape(B, Hkv, G, D).sum(axis=2)
    np.testing.assert_allclose(r["dV"].sum(axis=2), expect, atol=1e-12)
    # Delta (defined as sum_j P dP) equals rowsum(dO * O)
    np.testing.assert_allclose(r["Delta"], (do * r["O"]).sum(-1), atol=1e-12,
                               rtol=1e-12)


# --------------------------------------------------------------------------
# masks: brute force of the page's mask functions, TTT step-by-step form

def _page_causal(q_idx, kv_idx, shift, seq_len):
    return (q_idx - shift >= kv_idx) and (kv_idx < seq_len)


def _page_suffix(q_idx, kv_idx, q_len, seq_len):
    return (kv_idx >= q_len) and (kv_idx % q_len < seq_len) and \
        ((kv_idx - q_idx) % q_len == 0)


@pytest.mark.parametrize("L,steps,shift,seq", [(4, 1, 0, 4), (5, 3, 0, 5),
                                               (6, 3, 2, 4), (7, 2, 1, 7),
                                               (3, 4, 0, 2)])
def test_mask_predicate_brute_force(L, steps, shift, seq):
    Skv = L * steps
    A = allowed(TTT, L, Skv, shift, seq)
    C = allowed(CAUSAL, L, Skv, shift, seq)
    F = allowed(FULL, L, Skv, 0, seq)
    for i in range(L):
        for j in range(Skv):
            c = _page_causal(i, j, shift, seq)
            assert A[i, j] == (c or _page_suffix(i, j, L, seq)), (i, j)
            assert C[i, j] == c, (i, j)
            assert F[i, j] == (j < seq), (i, j)
    assert allowed_pair_count(TTT, L, Skv, shift, seq) == int(A.sum())


@pytest.mark.parametrize("t,shift,kvv", [(0, 0, None), (1, 0, None),
                                         (2, 0, None), (2, 2, None),
                                         (1, 1, (5, 3)), (2, 0, (7, 2))])
@pytest.mark.parametrize("L", [7, 16])
def test_ttt_predicate_equals_stepwise(L, t, shift, kvv):
    if kvv is not None:
        kvv = tuple(min(x, L) for x in kvv)
    B = 1 if kvv is None else len(kvv)
    Hq, Hkv, D = 4, 2, 8
    g = torch.Generator().manual_seed(L * 10 + t)
    q = torch.randn(B, Hq, L, D, generator=g, dtype=torch.float64, requires_grad=True)
    ks = [torch.randn(B, Hkv, L, D, generator=g, dtype=torch.float64,
                      requires_grad=True) for _ in range(t + 1)]
    vs = [torch.randn(B, Hkv, L, D, generator=g, dtype=torch.float64,
                      requires_grad=True) for _ in range(t + 1)]
    do = torch.randn(B, Hq, L, D, generator=g, dtype=torch.float64)
    O_s, LSE_s = ttt_stepwise_forward(q, ks, vs, shift, kvv)
    (O_s * do).sum().backward()

    kcat = torch.cat(ks, dim=2).detach().numpy()
    vcat = torch.cat(vs, dim=2).detach().numpy()
    r = attention_ref(q.detach().numpy(), kcat, vcat, do.numpy(), TTT, shift, kvv)
    np.testing.assert_allclose(r["O"], O_s.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(r["LSE"], LSE_s.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dQ"], q.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(r["dK"], torch.cat([x.grad for x in ks], 2).numpy(),
                               atol=1e-11)
    np.testing.assert_allclose(r["dV"], torch.cat([x.grad for x in vs], 2).numpy(),
                               atol=1e-11)


# --------------------------------------------------------------------------
# padding, empty rows, masked columns

def test_padding_equals_truncation_and_padded_grads_are_zero():
    B, H, Sq, Skv, D = 2, 2, 9, 12, 8
    q, k, v, do = (_rand((B, H, Sq, D), 50), _rand((B, H, Skv, D), 51),
                   _rand((B, H, Skv, D), 52), _rand((B, H, Sq, D), 53))
    kvv = (10, 5)
    r = attention_ref(q, k, v, do, FULL, 0, kvv)
    for b, n in enumerate(kvv):
        t = attention_ref(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n],
                          do[b:b + 1], FULL)
        for name in ("O", "LSE", "dQ"):
            np.testing.assert_allclose(r[name][b], t[name][0], atol=1e-13)
        np.testing.assert_allclose(r["dK"][b, :, :n], t["dK"][0], atol=1e-13)
        np.testing.assert_allclose(r["dV"][b, :, :n], t["dV"][0], atol=1e-13)
        assert np.all(r["dK"][b, :, n:] == 0.0) and np.all(r["dV"][b, :, n:] == 0.0)


def test_empty_rows_are_zero():
    B, H, S, D = 1, 2, 8, 4
    q, k, v, do = (_rand((B, H, S, D), 60), _rand((B, H, S, D), 61),
                   _rand((B, H, S, D), 62), _rand((B, H, S, D), 63))
    shift = 3
    r = attention_ref(q, k, v, do, CAUSAL, shift)
    assert np.all(r["O"][:, :, :shift] == 0.0)
    assert np.all(r["LSE"][:, :, :shift] == 0.0)
    assert np.all(r["dQ"][:, :, :shift] == 0.0)
    # keys j > S-1-shift are never attended: exactly zero gradient
    assert np.all(r["dK"][:, :, S - shift:] == 0.0)
    assert np.all(r["dV"][:, :, S - shift:] == 0.0)
    # the other rows equal causal attention of row i over keys 0..i-shift
    for i in range(shift, S):
        t = attention_forward(q[:, :, i:i + 1], k[:, :, : i - shift + 1],
                              v[:, :, : i - shift + 1], FULL)
        np.testing.assert_allclose(r["O"][:, :, i], t[0][:, :, 0], atol=1e-13)


def test_pair_counts_closed_form():
    S = 37
    assert allowed_pair_count(CAUSAL, S, S) == S * (S + 1) // 2
    assert allowed_pair_count(FULL, S, 20, 0, 13) == S * 13
    t = 2
    assert allowed_pair_count(TTT, S, (t + 1) * S) == S * (S + 1) // 2 + t * S
    # causal window of w + 1 keys: rows i < w see i + 1 keys, the rest w + 1
    w = 9
    assert allowed_pair_count(WINDOW, S, S, window=(w, 0)) == w * (w + 1) // 2 + (S - w) * (w + 1)
    # symmetric band of half-width w: (2w + 1) S minus the two clipped corners
    assert allowed_pair_count(WINDOW, S, S, window=(w, w)) == (2 * w + 1) * S - w * (w + 1)


# --------------------------------------------------------------------------
# WINDOW

def _band(Sq, Skv, shift, left, right):
    """Boolean band mask from torch.tril / torch.triu: j - i within
    [-shift - left, -shift + right]."""
    ones = torch.ones(Sq, Skv, dtype=torch.bool)
    return ones.tril(right - shift) & ones.triu(-shift - left)


@pytest.mark.parametrize("Hq,Hkv,Sq,Skv,shift,left,right", [
    (2, 2, 16, 16, 0, 3, 0), (4, 2, 13, 13, 0, 2, 2), (8, 1, 20, 20, 2, 5, 1),
    (2, 1, 12, 17, 0, 4, 6)])
def test_window_matches_torch_sdpa_band_mask(Hq, Hkv, Sq, Skv, shift, left, right):
    B, D = 2, 8
    q, k, v = _rand((B, Hq, Sq, D), 70), _rand((B, Hkv, Skv, D), 71), _rand((B, Hkv, Skv, D), 72)
    do = _rand((B, Hq, Sq, D), 73)
    band = _band(Sq, Skv, shift, left, right)
    rows = band.any(1).numpy()                    # SDPA gives NaN on empty rows
    assert rows.sum() >= Sq - shift
    r = attention_ref(q, k, v, do, WINDOW, shift, window=(left, right))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[:, :, rows], tk, tv, attn_mask=band[rows], enable_gqa=Hq != Hkv)
    out.backward(torch.tensor(do[:, :, rows]))
    np.testing.assert_allclose(r["O"][:, :, rows], out.detach().numpy(), atol=1e-12)
    assert np.all(r["O"][:, :, ~rows] == 0.0)
    np.testing.assert_allclose(r["dQ"][:, :, rows], tq.grad.numpy()[:, :, rows], atol=1e-11)
    for name, t in (("dK", tk), ("dV", tv)):
        assert np.abs(t.grad.numpy()).max() > 1e-3
        np.testing.assert_allclose(r[name], t.grad.numpy(), atol=1e-11, err_msg=name)


def test_window_limits_are_causal_and_full():
    B, Hq, Hkv, S, D = 1, 4, 2, 19, 8
    q, k, v = _rand((B, Hq, S, D), 80), _rand((B, Hkv, S, D), 81), _rand((B, Hkv, S, D), 82)
    do = _rand((B, Hq, S, D), 83)
    for shift in (0, 2):
        a = attention_ref(q, k, v, do, WINDOW, shift, (15,), window=(S, 0))
        c = attention_ref(q, k, v, do, CAUSAL, shift, (15,))
        for name in a:
            np.testing.assert_array_equal(a[name], c[name], err_msg=name)
    a = attention_ref(q, k, v, do, WINDOW, 0, (11,), window=(S, S))
    f = attention_ref(q, k, v, do, FULL, 0, (11,))
    for name in a:
        np.testing.assert_array_equal(a[name], f[name], err_msg=name)


def test_window_predicate_brute_force():
    Sq, Skv, shift, left, right, seq = 9, 13, 1, 2, 3, 11
    A = allowed(WINDOW, Sq, Skv, shift, seq, window=(left, right))
    for i in range(Sq):
        for j in range(Skv):
            expect = (i - shift - left <= j <= i - shift + right) and j < seq
            assert A[i, j] == expect, (i, j)


# --------------------------------------------------------------------------
# Prefix: CAUSAL with a negative shift -P (every query sees P prefix keys,
# then the causal part behind them)

@pytest.mark.parametrize("Hq,Hkv,Sq,P", [(2, 2, 11, 5), (4, 2, 16, 16), (8, 1, 9, 1)])
def test_prefix_matches_torch_sdpa_block_mask(Hq, Hkv, Sq, P):
    # the mask built as blocks: ones for the prefix columns beside a
    # lower-triangular block for the sequence (torch.ones, torch.tril)
    B, D = 2, 8
    Skv = P + Sq
    q, k, v = _rand((B, Hq, Sq, D), 90), _rand((B, Hkv, Skv, D), 91), _rand((B, Hkv, Skv, D), 92)
    do = _rand((B, Hq, Sq, D), 93)
    mask = torch.cat([torch.ones(Sq, P, dtype=torch.bool), torch.ones(Sq, Sq, dtype=torch.bool).tril()], dim=1)
    r = attention_ref(q, k, v, do, CAUSAL, -P)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, enable_gqa=Hq != Hkv)
    out.backward(torch.tensor(do))
    np.testing.assert_allclose(r["O"], out.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(r["dQ"], tq.grad.numpy(), atol=1e-11)
    for name, t in (("dK", tk), ("dV", tv)):
        assert np.abs(t.grad.numpy()[:, :, :P]).max() > 1e-3   # the prefix keys get gradient
        np.testing.assert_allclose(r[name], t.grad.numpy(), atol=1e-11, err_msg=name)
    # the predicate, pair by pair: j < P, or j - P <= i
    A = allowed(CAUSAL, Sq, Skv, -P)
    for i in range(Sq):
        for j in range(Skv):
            assert A[i, j] == (j < P or j - P <= i), (i, j)
    assert allowed_pair_count(CAUSAL, Sq, Skv, -P) == Sq * P + Sq * (Sq + 1) // 2


# --------------------------------------------------------------------------
# The key-range gradient (attention_key_grads), which the full-size parity
# tests use to check dK/dV of sampled key blocks over every attending row

def _torch_mask(kind, Sq, Skv, shift, kvv, window):
    """The allowed-pair matrix built from torch.tril / torch.triu / torch.eye
    and a column bound (not from the oracle's predicate)."""
    cols = torch.arange(Skv)[None, :]
    if kind == FULL:
        return (cols < kvv).expand(Sq, Skv).clone()
    if kind == WINDOW:
        return _band(Sq, Skv, shift, *window) & (cols < kvv)
    tri = torch.ones(Sq, Skv, dtype=torch.bool).tril(-shift)
    if kind == CAUSAL:
        return tri & (cols < kvv)
    L = Sq   # TTT: the causal step-0 block, then one diagonal per later step
    blocks = [tri[:, :L] & (cols[:, :L] < kvv)]
    rows_ok = (torch.arange(L) < kvv)[:, None]
    for _ in range(1, Skv // L):
        blocks.append(torch.eye(L, dtype=torch.bool) & rows_ok)
    return torch.cat(blocks, dim=1)


@pytest.mark.parametrize("kind,Sq,Skv,shift,kvv,win,keys", [
    (CAUSAL, 24, 24, 0, (24, 17), None, (5, 13)),
    (CAUSAL, 20, 30, -10, (30, 30), None, (0, 12)),      # a prefix before the diagonal
    (FULL, 16, 21, 0, (21, 9), None, (7, 21)),
    (TTT, 12, 36, 0, (12, 7), None, (8, 30)),
    (TTT, 10, 30, 2, (10, 10), None, (0, 30)),
    (WINDOW, 22, 22, 1, (22, 15), (4, 2), (3, 19)),
])
def test_key_grads_match_torch_sdpa_autograd(kind, Sq, Skv, shift, kvv, win, keys):
    from oracle import attention_key_grads
    B, Hq, Hkv, D = 2, 4, 2, 8
    q, k, v = _rand((B, Hq, Sq, D), 100), _rand((B, Hkv, Skv, D), 101), _rand((B, Hkv, Skv, D), 102)
    do = _rand((B, Hq, Sq, D), 103)
    dK, dV = attention_key_grads(q, k, v, do, keys, kind, shift, kvv, window=win)
    k0, k1 = keys
    for b in range(B):
        mask = _torch_mask(kind, Sq, Skv, shift, kvv[b], win)
        rows = mask.any(1)                     # SDPA gives NaN on rows with no key
        tq, tk, tv = (torch.tensor(x[b:b + 1], requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(
            tq[:, :, rows], tk, tv, attn_mask=mask[rows], enable_gqa=True)
        out.backward(torch.tensor(do[b:b + 1][:, :, rows.numpy()]))
        gk, gv = tk.grad.numpy()[0, :, k0:k1], tv.grad.numpy()[0, :, k0:k1]
        assert np.abs(gk).max() > 1e-3 and np.abs(gv).max() > 1e-3
        np.testing.assert_allclose(dK[b], gk, atol=1e-11, err_msg=f"dK b={b}")
        np.testing.assert_allclose(dV[b], gv, atol=1e-11, err_msg=f"dV b={b}")


# --------------------------------------------------------------------------
# The per-batch key bias (the additive mask of the playbook's "3. Per-trainer
# porting checklist", in its [B, Skv] form): bias[b, j] is added to the
# scaled score of every row and head of batch entry b with key j.

def _bias(B, Skv, seed, neg_inf_frac=0.15):
    """Finite biases in [-3, 3] with some -inf entries (never a whole row)."""
    g = np.random.default_rng(seed)
    b = g.uniform(-3.0, 3.0, (B, Skv))
    drop = g.uniform(size=(B, Skv)) < neg_inf_frac
    drop[:, 0] = False
    b[drop] = -np.inf
    return b


@pytest.mark.parametrize("kind,Sq,Skv,shift,win", [
    (FULL, 18, 23, 0, None),
    (CAUSAL, 20, 20, 0, None),
    (CAUSAL, 16, 26, -10, None),
    (WINDOW, 22, 22, 1, (4, 2)),
])
def test_bias_neg_inf_tail_equals_kv_valid(kind, Sq, Skv, shift, win):
    # a bias that is 0 on keys below n and -inf from n on is the padding
    # mask kv_valid = n: the same allowed pairs with the same scores, so every
    # output is bitwise the same
    B, Hq, Hkv, D = 2, 4, 2, 8
    q, k, v = _rand((B, Hq, Sq, D), 120), _rand((B, Hkv, Skv, D), 121), _rand((B, Hkv, Skv, D), 122)
    do = _rand((B, Hq, Sq, D), 123)
    kvv = (Skv - 5, 7)
    bias = np.zeros((B, Skv))
    for b in range(B):
        bias[b, kvv[b]:] = -np.inf
    a = attention_ref(q, k, v, do, kind, shift, kvv, window=win)
    c = attention_ref(q, k, v, do, kind, shift, None, window=win, bias=bias)
    for name in ("O", "LSE", "dQ", "dK", "dV", "Delta"):
        np.testing.assert_array_equal(a[name], c[name], err_msg=name)


@pytest.mark.parametrize("kind", [FULL, CAUSAL, TTT])
def test_bias_constant_shifts_lse_only(kind):
    # softmax is unchanged by adding one constant to a row's scores: O and the
    # gradients stay, LSE moves by the constant
    B, Hq, Hkv, Sq, D = 2, 4, 2, 12, 8
    Skv = 3 * Sq if kind == TTT else Sq
    q, k, v = _rand((B, Hq, Sq, D), 130), _rand((B, Hkv, Skv, D), 131), _rand((B, Hkv, Skv, D), 132)
    do = _rand((B, Hq, Sq, D), 133)
    c = np.array([[2.5] * Skv, [-7.25] * Skv])
    a = attention_ref(q, k, v, do, kind)
    r = attention_ref(q, k, v, do, kind, bias=c)
    for name in ("O", "dQ", "dK", "dV", "Delta"):
        np.testing.assert_allclose(r[name], a[name], atol=1e-12, err_msg=name)
    np.testing.assert_allclose(r["LSE"], a["LSE"] + c[:, 0][:, None, None], atol=1e-12)


@pytest.mark.parametrize("kind,Sq,Skv,shift,win", [
    (FULL, 17, 29, 0, None),
    (CAUSAL, 24, 24, 0, None),
    (CAUSAL, 20, 30, -10, None),
    (TTT, 12, 36, 0, None),
    (WINDOW, 22, 22, 1, (4, 2)),
])
def test_bias_matches_torch_sdpa_float_mask(kind, Sq, Skv, shift, win):
    # torch's SDPA with a float attn_mask (the bias where the kind allows the
    # pair, -inf elsewhere) against the oracle: O, and dQ, dK, dV by autograd
    B, Hq, Hkv, D = 2, 4, 2, 8
    q, k, v = _rand((B, Hq, Sq, D), 140), _rand((B, Hkv, Skv, D), 141), _rand((B, Hkv, Skv, D), 142)
    do = _rand((B, Hq, Sq, D), 143)
    bias = _bias(B, Skv, 144)
    r = attention_ref(q, k, v, do, kind, shift, None, window=win, bias=bias)
    for b in range(B):
        allow = _torch_mask(kind, Sq, Skv, shift, Skv if kind != TTT else Sq, win)
        fmask = torch.where(allow, torch.tensor(bias[b])[None, :].expand(Sq, Skv),
                            torch.tensor(-np.inf, dtype=torch.float64))
        rows = torch.isfinite(fmask).any(1)   # SDPA gives NaN on rows with no key
        tq, tk, tv = (torch.tensor(x[b:b + 1], requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(
            tq[:, :, rows], tk, tv, attn_mask=fmask[rows], enable_gqa=True)
        out.backward(torch.tensor(do[b:b + 1][:, :, rows.numpy()]))
        np.testing.assert_allclose(r["O"][b][:, rows.numpy()], out.detach().numpy()[0], atol=1e-12)
        assert np.all(r["O"][b][:, ~rows.numpy()] == 0) and np.all(r["LSE"][b][:, ~rows.numpy()] == 0)
        np.testing.assert_allclose(r["dQ"][b], tq.grad.numpy()[0], atol=1e-11, err_msg="dQ")
        np.testing.assert_allclose(r["dK"][b], tk.grad.numpy()[0], atol=1e-11, err_msg="dK")
        np.testing.assert_allclose(r["dV"][b], tv.grad.numpy()[0], atol=1e-11, err_msg="dV")
        # LSE: the natural logsumexp of the biased scores over allowed keys
        S = (q[b] @ np.repeat(k[b], Hq // Hkv, 0).transpose(0, 2, 1)) / np.sqrt(D)
        L = torch.logsumexp(torch.tensor(S) + fmask[None], dim=-1).numpy()
        np.testing.assert_allclose(r["LSE"][b][:, rows.numpy()], L[:, rows.numpy()], atol=1e-12)


def test_bias_key_grads_match_full_backward():
    from oracle import attention_key_grads
    B, Hq, Hkv, Sq, Skv, D = 2, 4, 2, 20, 20, 8
    q, k, v = _rand((B, Hq, Sq, D), 150), _rand((B, Hkv, Skv, D), 151), _rand((B, Hkv, Skv, D), 152)
    do = _rand((B, Hq, Sq, D), 153)
    bias = _bias(B, Skv, 154)
    r = attention_ref(q, k, v, do, CAUSAL, bias=bias)
    dK, dV = attention_key_grads(q, k, v, do, (4, 15), CAUSAL, bias=bias)
    np.testing.assert_allclose(dK, r["dK"][:, :, 4:15], atol=1e-12)
    np.testing.assert_allclose(dV, r["dV"][:, :, 4:15], atol=1e-12)
