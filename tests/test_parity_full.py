"""GPU parity at the workloads' full sizes, through the same calls the
benchmark times (fa_fwd, then fa_bwd).

The fp64 oracle cannot materialise 16K x 16K scores for every head, so each
case compares what it can compute exactly:

* one-head groups (Hq == Hkv: the batch-8 grid and the diffusion-transformer
  shapes): every output of sampled (batch, head) pairs, whole;
* grouped long-context and TTT shapes: O, LSE and dQ of sampled query-row
  blocks (first, middle and last 64 rows) for every head of a sampled K/V
  group, and dK, dV of the keys that only those rows may attend (for the last
  block that is the final keys of the causal part and, under TTT, the later
  steps' keys at those positions), all exact;
* grouped shapes again: dK, dV of sampled 256-key blocks (an early one, at
  an eighth of the sequence, and a middle one; under TTT also a block of the
  step-1 keys) element by element, from the oracle over every query row that
  attends them, in every head of the group;
* everywhere: two identities that hold at any size for every (batch, K/V
  head): the dK rows sum to zero (each softmax-gradient row dS_i sums to zero)
  and the dV rows sum to the dO rows of the group's non-empty query rows (each
  P row sums to one).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import flash_attention_fa_amd as fa
import workloads as W
from oracle import allowed, attention_key_grads, attention_ref
from parity_util import TOL_BF16, TOL_LSE_BF16, say

pytestmark = pytest.mark.gpu

ROWS = 64


def run_like_bench(w, q, k, v, do):
    dev = "cuda"
    qg, kg, vg, dog = (x.to(dev) for x in (q, k, v, do))
    kvv = W.kv_valid_tensor(w, dev)
    kw = dict(mask_kind=w.kind, causal_shift=w.shift, kv_valid=kvv, scale=w.scale, window=w.window,
              frozen_keys=w.frozen)
    o, lse = fa.fa_fwd(qg, kg, vg, **kw)
    dq, dk, dv = torch.empty_like(qg), torch.empty_like(kg), torch.empty_like(vg)
    ws = torch.empty(max(1, fa.fa_bwd_workspace_bytes(qg, kg, mask_kind=w.kind)), dtype=torch.uint8, device=dev)
    fa.fa_bwd(qg, kg, vg, o, lse, dog, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    scale = float(np.abs(ref).max())
    assert scale > 0, "reference is all zero (vacuous)"
    return float(np.abs(got - ref).max()) / scale


def kvv_of(w, b):
    return None if w.kv_valid is None else w.kv_valid[b]


def check_identities(w, do, o, dk, dv, label):
    """sum_j dK_j = 0 and sum_j dV_j = sum over non-empty rows of dO, per (b, kv head).
    With frozen keys (their dK, dV left at zero) the sums are not over all
    keys, so the check is that the frozen rows are exactly zero instead."""
    if w.frozen:
        assert torch.all(dk[:, :, :w.frozen] == 0) and torch.all(dv[:, :, :w.frozen] == 0), \
            f"{label}: frozen keys must hold exactly zero dK, dV"
        return
    G = w.Hq // w.Hkv
    for b in range(w.B):
        # a row is empty iff no key is allowed; with these masks (valid keys
        # from 0, causal shift s) only rows below s can be
        nonempty = np.ones(w.Sq, bool)
        probe = np.arange(min(w.Sq, 64 + w.shift))
        nonempty[probe] = allowed(w.kind, w.Sq, w.Skv, w.shift, kvv_of(w, b), rows=probe,
                                  window=w.window).any(1)
        for g in range(w.Hkv):
            dk_bg = f64(dk[b, g])
            dv_bg = f64(dv[b, g])
            do_grp = f64(do[b, g * G:(g + 1) * G]).reshape(-1, w.D)
            target = do_grp.reshape(G, w.Sq, w.D)[:, nonempty].sum(axis=(0, 1))
            mag_k = np.abs(dk_bg).sum(axis=0).max()
            mag_v = np.abs(dv_bg).sum(axis=0).max()
            assert mag_k > 0 and mag_v > 0, f"{label} b={b} g={g}: vacuous gradients"
            ek = np.abs(dk_bg.sum(axis=0)).max() / mag_k
            ev = np.abs(dv_bg.sum(axis=0) - target).max() / mag_v
            assert ek <= 1e-2, f"{label} b={b} g={g}: |sum dK| / sum|dK| = {ek:.2e}"
            assert ev <= 1e-2, f"{label} b={b} g={g}: sum dV vs sum dO: {ev:.2e}"


def whole_head_cases():
    return [w for w in W.all_workloads() if w.dtype == "bf16" and w.Hq == w.Hkv]


@pytest.mark.parametrize("w", whole_head_cases(), ids=lambda w: w.name)
def test_full_size_whole_heads(w):
    """Every output of sampled (batch, head) pairs against the oracle."""
    say(f"[full] {w.name} B={w.B} H={w.Hq} Sq={w.Sq} Skv={w.Skv} D={w.D}")
    q, k, v, do = W.make_inputs(w, seed=1)
    o, lse, dq, dk, dv = run_like_bench(w, q, k, v, do)
    samples = sorted({(0, 0), (w.B - 1, w.Hq - 1), (w.B // 2, w.Hq // 2)})
    for b, h in samples:
        sl = lambda x: x[b:b + 1, h:h + 1].double().numpy()
        ref = attention_ref(sl(q), sl(k), sl(v), sl(do), w.kind, w.shift,
                            None if w.kv_valid is None else [w.kv_valid[b]], w.scale, window=w.window)
        got = dict(O=o[b, h], LSE=lse[b, h], dQ=dq[b, h], dK=dk[b, h], dV=dv[b, h])
        errs = {}
        for name, g in got.items():
            r = ref[name][0, 0]
            gg = f64(g)
            if name == "LSE":
                errs[name] = float(np.abs(gg - r).max())
                assert errs[name] <= TOL_LSE_BF16, f"{w.name} ({b},{h}) LSE {errs[name]:.2e}"
            else:
                if name in ("dK", "dV") and w.kv_valid is not None:
                    n = w.kv_valid[b]
                    assert np.all(gg[n:] == 0), f"{w.name} ({b},{h}) {name}: padded keys not zero"
                    gg, r = gg[:n], r[:n]
                errs[name] = rel_err(gg, r)
                assert errs[name] <= TOL_BF16[name], f"{w.name} ({b},{h}) {name} {errs[name]:.2e}"
        say(f"[full] {w.name} (b={b}, h={h}) ok {errs}")
    check_identities(w, do, o, dk, dv, w.name)


def grouped_cases():
    return [w for w in W.all_workloads() if w.dtype == "bf16" and w.Hq != w.Hkv]


def complete_keys(w, b, lo, hi):
    """Keys every one of whose attending query rows lies in [lo, hi).

    Candidates are the keys at positions (mod Sq) from lo - shift - 1 on;
    rows far below lo are not scanned (under causal, TTT and right-closed
    window masks they see no such key).  Were that wrong, the oracle's dK/dV of a key would miss
    contributions and the comparison would fail, never pass falsely."""
    L = w.Sq
    cand = np.arange(w.Skv)
    pos = cand % L if w.kind == W.TTT else cand
    cand = cand[pos >= max(0, lo - w.shift - 1)]
    outside = np.concatenate([np.arange(max(0, lo - max(w.shift, 0) - 256), lo), np.arange(hi, w.Sq)])
    seen = np.zeros(len(cand), bool)
    for r0 in range(0, len(outside), 2048):
        A = allowed(w.kind, w.Sq, w.Skv, w.shift, kvv_of(w, b), rows=outside[r0:r0 + 2048], window=w.window)
        seen |= A[:, cand].any(0)
    inside = allowed(w.kind, w.Sq, w.Skv, w.shift, kvv_of(w, b), rows=np.arange(lo, hi),
                     window=w.window)[:, cand].any(0)
    return cand[~seen & inside]


@pytest.mark.parametrize("w", grouped_cases(), ids=lambda w: w.name)
def test_full_size_grouped_row_samples(w):
    """Sampled row blocks of one K/V group, and the keys only they attend."""
    say(f"[full] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Sq={w.Sq} Skv={w.Skv} D={w.D}")
    q, k, v, do = W.make_inputs(w, seed=1)
    o, lse, dq, dk, dv = run_like_bench(w, q, k, v, do)
    G = w.Hq // w.Hkv
    b, g = w.B - 1, w.Hkv - 1
    hs = slice(g * G, (g + 1) * G)
    qs, ks, vs, dos = (x[b:b + 1, hs if i in (0, 3) else slice(g, g + 1)].double().numpy()
                       for i, x in enumerate((q, k, v, do)))
    kvv = None if w.kv_valid is None else [w.kv_valid[b]]
    blocks = [(0, ROWS), (w.Sq // 2 - ROWS // 2, w.Sq // 2 + ROWS // 2), (w.Sq - ROWS, w.Sq)]
    for lo, hi in blocks:
        ref = attention_ref(qs, ks, vs, dos, w.kind, w.shift, kvv, w.scale, rows=(lo, hi), window=w.window)
        errs = {}
        for name, got in (("O", o), ("dQ", dq)):
            errs[name] = rel_err(f64(got[b, hs, lo:hi]), ref[name][0, :, lo:hi])
            assert errs[name] <= TOL_BF16[name], f"{w.name} rows [{lo},{hi}) {name} {errs[name]:.2e}"
        errs["LSE"] = float(np.abs(f64(lse[b, hs, lo:hi]) - ref["LSE"][0, :, lo:hi]).max())
        assert errs["LSE"] <= TOL_LSE_BF16, f"{w.name} rows [{lo},{hi}) LSE {errs['LSE']:.2e}"
        # only the last block owns keys outright (every earlier key is seen
        # by the rows after it)
        keys = complete_keys(w, b, lo, hi) if hi == w.Sq else []
        if len(keys):
            for name, got in (("dK", dk), ("dV", dv)):
                errs[name] = rel_err(f64(got[b, g])[keys], ref[name][0, 0][keys])
                assert errs[name] <= TOL_BF16[name], f"{w.name} keys of [{lo},{hi}) {name} {errs[name]:.2e}"
        say(f"[full] {w.name} rows [{lo},{hi}) complete keys {len(keys)} ok {errs}")
        if (lo, hi) == blocks[-1]:
            assert len(keys) >= ROWS // 2, "the last row block should own some keys outright"
    check_identities(w, do, o, dk, dv, w.name)


KEY_BLOCK = 256


def sampled_key_blocks(w):
    """An early and a middle 256-key block of the walked keys (past a frozen
    prefix, whose gradients are exact zeros and checked as such), and under
    TTT a block of the step-1 keys."""
    L = w.Sq if w.kind == W.TTT else w.Skv
    base = w.frozen
    span = L - base
    starts = [base + (span // 8) // KEY_BLOCK * KEY_BLOCK, base + (span // 2) // KEY_BLOCK * KEY_BLOCK]
    if w.kind == W.TTT:
        starts.append(w.Sq + (w.Sq // 2) // KEY_BLOCK * KEY_BLOCK)
    return [(s, min(w.Skv, s + KEY_BLOCK)) for s in starts]


def oracle_key_block(w, q, k, v, do, b, g, keys):
    """dK, dV of keys [k0, k1) of (b, K/V head g) from the oracle, one query
    head per worker thread (the group's heads summed in order afterwards)."""
    G = w.Hq // w.Hkv
    kvv = None if w.kv_valid is None else [w.kv_valid[b]]
    K, V = (x[b:b + 1, g:g + 1].double().numpy() for x in (k, v))

    def one(h):
        Q, DO = (x[b:b + 1, h:h + 1].double().numpy() for x in (q, do))
        return attention_key_grads(Q, K, V, DO, keys, w.kind, w.shift, kvv, w.scale, window=w.window)

    with threadpool_limits(limits=2), ThreadPoolExecutor(max_workers=G) as ex:
        parts = list(ex.map(one, range(g * G, (g + 1) * G)))
    dK = sum(p[0][0, 0] for p in parts)
    dV = sum(p[1][0, 0] for p in parts)
    return dK, dV


@pytest.mark.parametrize("w", grouped_cases(), ids=lambda w: w.name)
def test_full_size_grouped_key_blocks(w):
    """dK, dV of sampled key blocks of one K/V group, element by element,
    against the oracle over every query row (of every head of the group) that
    attends them."""
    say(f"[full] {w.name} key blocks {sampled_key_blocks(w)}")
    q, k, v, do = W.make_inputs(w, seed=1)
    o, lse, dq, dk, dv = run_like_bench(w, q, k, v, do)
    b, g = w.B - 1, 0
    for k0, k1 in sampled_key_blocks(w):
        rk, rv = oracle_key_block(w, q, k, v, do, b, g, (k0, k1))
        errs = {}
        for name, got, ref in (("dK", dk, rk), ("dV", dv, rv)):
            errs[name] = rel_err(f64(got[b, g, k0:k1]), ref)
            assert errs[name] <= TOL_BF16[name], f"{w.name} keys [{k0},{k1}) {name} {errs[name]:.2e}"
        say(f"[full] {w.name} keys [{k0},{k1}) ok {errs}")


def test_peak_memory_linear_in_S():
    """fa_fwd + fa_bwd allocate nothing beyond their inputs, outputs and a
    workspace linear in S: the peak grows by 2x when S doubles."""
    peaks = []
    for S in (8192, 16384):
        w = W.long_gqa(S)
        q, k, v, do = (x.cuda() for x in W.make_inputs(w, seed=0))
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        o, lse = fa.fa_fwd(q, k, v, mask_kind=w.kind)
        dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, mask_kind=w.kind)
        torch.cuda.synchronize()
        inputs = sum(x.numel() * x.element_size() for x in (q, k, v, do))
        peaks.append(torch.cuda.max_memory_allocated() - base + inputs)
        del q, k, v, do, o, lse, dq, dk, dv
        torch.cuda.empty_cache()
    ratio = peaks[1] / peaks[0]
    say(f"[memory] peak bytes at S=8192, 16384: {peaks} ratio {ratio:.3f}")
    assert 1.95 <= ratio <= 2.05
