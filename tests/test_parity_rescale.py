"""GPU parity on inputs that make the bf16 forward rescale live accumulators.

The forward keeps a lazy running max per query row (the online-softmax
update of CS336 "Flash Attention (Triton)", How it works: the running max m
and normaliser l, with the accumulated output rescaled when m grows).  P of a
key tile is taken against a stored reference, and only when some lane's sum
of P over its 32 keys of the tile passes a bound does the wave take the true
tile max and rescale O and l.  Two forms, by head dim:

- D <= 32: the reference is a row max, the bound 4096 (= 2^12, so no P can
  overflow first); O and l are rescaled and P recomputed before the PV
  products.
- D >= 64: the reference is 2^12 above a row max and P saturates at 1, so
  the bound is a lane sum of 1; the PV products run first and the tile is
  corrected after them (O, l scaled by alpha = exp(m_old - m_new), then
  the difference between the new and the used P goes through the PV
  product).

With N(0, 1) inputs no tile after the first ever passes either bound, so the
rescale of accumulators that already hold values is reached only by inputs
built for it: the ``spike`` recipe of ``workloads.make_stress_inputs`` (flat
scores, then eight keys about 7 units higher in one lane half of one key
tile, with the mean of V flipped on them).

Before any GPU call, ``guaranteed_live_refreshes`` proves from the inputs
alone (fp64, on the CPU) that the branch is reached: the lazy max is never
above the true running max M of the keys a row has seen, so a lane whose
half-tile sum of exp(s - M) exceeds 4096 (with 5 % slack for rounding)
certainly triggers the refresh (at D >= 64 its sum of min(1, exp(s - m -
ln 4096)) with m <= M is then at least 1), and with M finite the row's
accumulators are live.  The test also requires that these rows carry at least 20 % of their
softmax mass in the rescaled accumulators and that V's mean differs in sign
between the keys before and at the spike, so a mistake in the rescale moves
O by a large fraction of max|O| and cannot pass the 2e-2 bar.

Also here: the untimed stress variants of peaky queries (Q x 4) and uniform
U(-1, 1) inputs, at the standard tolerances.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import allowed, attention_ref
from parity_util import TOL_BF16, TOL_LSE_BF16, check_case, run_gpu, say

FULL, CAUSAL, TTT, WINDOW = W.FULL, W.CAUSAL, W.TTT, W.WINDOW

TK = 64           # the forward's key tile
SUM_LIMIT = 4096.0
SPIKE_TILE_KEY = 3072
# eight keys that one lane half holds in the forward's score layout (offsets
# whose bit 2 is clear), so their sum alone decides that lane's refresh
SPIKES = tuple(SPIKE_TILE_KEY + o for o in (0, 1, 2, 3, 8, 9, 10, 11))
LEVEL = 7.0


def guaranteed_live_refreshes(q, k, kind, shift=0, window=None, b=0, h=0, slack=1.05, block=256):
    """Rows of (b, h) whose forward provably rescales live accumulators.

    Returns {row: mass fraction held by the accumulators at that rescale},
    taking the largest fraction when a row has several.  Walks each row's
    key tiles in the forward's order (increasing; under TTT the step-0 keys,
    after the later steps' keys, which the forward folds in first).  Rows are
    taken in blocks only to bound memory.
    """
    B, Hq, Sq, D = q.shape
    Skv = k.shape[2]
    G = Hq // k.shape[1]
    Kt = k[b, h // G].double().numpy().T
    nkeys = Sq if kind == TTT else Skv
    out = {}
    for r0 in range(0, Sq, block):
        rows = np.arange(r0, min(Sq, r0 + block))
        S = (q[b, h, rows].double().numpy() @ Kt) / np.sqrt(D)
        A = allowed(kind, Sq, Skv, shift, None, rows=rows, window=window)
        top = np.where(A, S, -np.inf).max(1)
        E = np.where(A, np.exp(np.minimum(S - top[:, None], 0.0)), 0.0)   # the final softmax, unnormalised
        total = E.sum(1)
        fold = A.copy()
        fold[:, :nkeys] = False
        M = np.where(fold.any(1), np.where(fold, S, -np.inf).max(1), -np.inf)   # true running max
        before = E[:, nkeys:].sum(1)
        best = np.full(len(rows), -1.0)
        for t in range((nkeys + TK - 1) // TK):
            ks = np.arange(t * TK, min(nkeys, (t + 1) * TK))
            a = A[:, ks]
            if not a.any():
                continue
            half = ((ks - t * TK) >> 2) & 1
            live = np.isfinite(M)
            with np.errstate(over="ignore", invalid="ignore"):
                x = np.where(a & live[:, None], np.exp(S[:, ks] - np.where(live, M, 0.0)[:, None]), 0.0)
            fires = np.zeros(len(rows), bool)
            for hh in (0, 1):
                fires |= x[:, half == hh].sum(1) > SUM_LIMIT * slack
            fires &= live
            best = np.where(fires, np.maximum(best, before / total), best)
            M = np.maximum(M, np.where(a, S[:, ks], -np.inf).max(1))
            before += E[:, ks].sum(1)
        out.update({int(rows[i]): float(best[i]) for i in np.nonzero(best >= 0)[0]})
    return out


def spike_inputs(B, Hq, Hkv, Sq, Skv, D, seed):
    return W.make_stress_inputs("spike", B, Hq, Hkv, Sq, Skv, D, seed=seed, spikes=SPIKES, level=LEVEL)


def assert_reaches_rescale(q, k, v, kind, window=None, heads=(0,), label=""):
    """The CPU proof that the case exercises the rescale, with teeth."""
    G = q.shape[1] // k.shape[1]
    for h in heads:
        ev = guaranteed_live_refreshes(q, k, kind, window=window, h=h)
        strong = [i for i, f in ev.items() if f >= 0.2]
        say(f"[rescale] {label} head {h}: {len(ev)} rows provably rescale live accumulators, "
            f"{len(strong)} of them holding >= 20 % of the row's mass")
        assert len(strong) >= 256, f"{label}: the inputs do not reach the rescale often enough"
    # V's mean differs in sign between the keys before the spike and the spike keys
    vv = v[0, h // G].float()
    before = vv[:SPIKES[0]].mean().item()
    at = vv[list(SPIKES)].mean().item()
    assert before > 0.5 and at < -0.5, (before, at)


CASES = [
    # name, kind, Sq, Skv, window
    ("causal", CAUSAL, 4096, 4096, None),
    ("ttt_t2", TTT, 4096, 3 * 4096, None),
    ("window", WINDOW, 4096, 4096, (3500, 0)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bf16_rescale_four_wave(case, D):
    """4-wave forward (128 query rows per workgroup: few workgroups), GQA."""
    name, kind, Sq, Skv, win = case
    q, k, v, do = spike_inputs(1, 2, 1, Sq, Skv, D, seed=200 + D)
    assert_reaches_rescale(q, k, v, kind, window=win, heads=(0, 1), label=f"{name} D={D}")
    check_case(q, k, v, do, kind, "bf16", window=win, label=f"bf16 rescale 4-wave {name} D={D}")


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bf16_rescale_eight_wave(case):
    """8-wave forward (B * Hq * ceil(Sq / 256) = 512 workgroups of 256 rows).
    One K/V head per query head, so sampled heads are checked whole."""
    name, kind, Sq, Skv, win = case
    D, H = 128, 32
    assert H * ((Sq + 255) // 256) >= 512
    q, k, v, do = spike_inputs(1, H, H, Sq, Skv, D, seed=300)
    sampled = (0, H - 1)
    assert_reaches_rescale(q, k, v, kind, window=win, heads=sampled, label=f"{name} 8-wave")
    say(f"[parity] bf16 rescale 8-wave {name} q{tuple(q.shape)} k{tuple(k.shape)}")
    got = run_gpu(q, k, v, do, kind, window=win)
    for h in sampled:
        sl = lambda x: x[:, h:h + 1].double().numpy()
        ref = attention_ref(sl(q), sl(k), sl(v), sl(do), kind, window=win)
        errs = {}
        for nm in ("O", "LSE", "dQ", "dK", "dV"):
            g, r = got[nm][:, h:h + 1], ref[nm]
            if nm == "LSE":
                errs[nm] = float(np.abs(g - r).max())
                assert errs[nm] <= TOL_LSE_BF16, f"{name} head {h} LSE {errs[nm]:.2e}"
            else:
                if nm in ("dK", "dV"):
                    seen = allowed(kind, Sq, Skv, 0, None, window=win).any(0)
                    assert np.all(g[:, :, ~seen] == 0), f"{name} head {h} {nm}: unattended keys not zero"
                    g, r = g[:, :, seen], r[:, :, seen]
                errs[nm] = float(np.abs(g - r).max()) / float(np.abs(r).max())
                assert errs[nm] <= TOL_BF16[nm], f"{name} head {h} {nm} {errs[nm]:.2e}"
        say(f"[parity] bf16 rescale 8-wave {name} head {h} ok {errs}")


STRESS = [
    # recipe, kind, B, Hq, Hkv, Sq, Skv, D
    ("peaky", CAUSAL, 1, 8, 2, 700, 700, 128),
    ("peaky", TTT, 1, 8, 2, 300, 900, 128),
    ("peaky", FULL, 2, 4, 4, 333, 333, 64),
    ("uniform", CAUSAL, 1, 8, 2, 700, 700, 128),
    ("uniform", WINDOW, 2, 4, 2, 333, 333, 64),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", STRESS, ids=[f"{c[0]}_{W.KIND_NAMES[c[1]]}_D{c[7]}" for c in STRESS])
def test_bf16_stress_inputs(case):
    recipe, kind, B, Hq, Hkv, Sq, Skv, D = case
    q, k, v, do = W.make_stress_inputs(recipe, B, Hq, Hkv, Sq, Skv, D, seed=400 + Sq)
    win = (100, 20) if kind == WINDOW else None
    check_case(q, k, v, do, kind, "bf16", window=win, label=f"bf16 stress {recipe} {W.KIND_NAMES[kind]} D={D}")


def test_spike_inputs_reach_the_rescale_on_cpu():
    """The guarantee itself, on the CPU (no GPU needed): the GPU cases above
    are built so that the rescale of live accumulators is provably reached."""
    for name, kind, Sq, Skv, win in CASES:
        q, k, v, do = spike_inputs(1, 2, 1, Sq, Skv, 128, seed=328)
        assert_reaches_rescale(q, k, v, kind, window=win, heads=(0,), label=name)


def test_normal_inputs_never_reach_the_rescale():
    """Why the spike recipe exists: on N(0, 1) inputs the bound is never
    provably passed after the first tile (so the older tests could not reach
    the rescale of live accumulators)."""
    g = torch.Generator("cpu").manual_seed(5)
    q, k = (torch.randn(1, 1, 2048, 128, generator=g).to(torch.bfloat16) for _ in range(2))
    assert guaranteed_live_refreshes(q, k, CAUSAL) == {}
