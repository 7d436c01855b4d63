"""GPU parity of the soft-target log-softmax loss (fa_lsm_loss_fwd / _bwd)
against the fp64 oracle on the same float32 inputs.

Tolerances, derived from float32 arithmetic (the library computes in fp32):
  * m (the row max) is exact;
  * d, tsum: relative error <= 1e-5;
  * row loss: |err| <= 2e-5 * sum_v |t_iv| (|x_iv| + |lse_i|) + 1e-6, the
    magnitude of the summands of the row's sum (cancellation between
    sum t x and lse * tsum is allowed for);
  * the mean loss: the same bound averaged over rows;
  * the gradient: per row, max |err| <= 1e-5 * max |ref| + 1e-12.
Masked rows (weight 0) must hold exactly row = 0 and gradient = 0.
"""
import numpy as np
import pytest
import torch

import flash_attention_fa_amd as fa
import workloads as W
from oracle import logsoftmax_loss_forward as lfwd, logsoftmax_loss_backward as lbwd

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def np64(t):
    return t.detach().cpu().double().numpy()


def check(x, t, w, xg_out, got, grad_loss=1.0, rows=None):
    """x, t, w: the float32 inputs (CPU); got: (loss, row, m, d, tsum) from the
    library; xg_out: the gradient it wrote; rows: row indices to compare
    (None = all, and the mean is compared too)."""
    loss, row, m, d, tsum = (np64(a) for a in got)
    X, T = np64(x), np64(t)
    Wt = None if w is None else np64(w)
    idx = np.arange(X.shape[0]) if rows is None else np.asarray(rows)
    Xs, Ts = X[idx], T[idx]
    ws = None if Wt is None else Wt[idx]
    _, rref, mref, dref, tref = lfwd(Xs, Ts, ws)
    lse = mref + np.log(dref)
    scale = (np.abs(Ts) * (np.abs(Xs) + np.abs(lse)[:, None])).sum(axis=1)
    assert np.array_equal(m[idx], mref), "row max"
    assert np.abs(d[idx] / dref - 1).max() <= 1e-5
    assert np.abs(tsum[idx] - tref).max() <= 1e-5 * np.abs(tref).max() + 1e-30
    err = np.abs(row[idx] - rref)
    assert np.all(err <= 2e-5 * scale * (1 if ws is None else np.abs(ws)) + 1e-6), err.max()
    # the gradient of the rows, with the mean over all N rows
    N = X.shape[0]
    gref = lbwd(Xs, Ts, ws, grad_loss=grad_loss) * len(idx) / N
    G = np64(xg_out)[idx]
    gerr = np.abs(G - gref).max(axis=1)
    assert np.all(gerr <= 1e-5 * np.abs(gref).max(axis=1) + 1e-12), gerr.max()
    if ws is not None:
        z = ws == 0
        assert np.all(row[idx][z] == 0) and np.all(G[z] == 0)
    if rows is None:
        full = rref.sum() / N
        assert abs(loss[0] - full) <= 2e-5 * scale.mean() + 1e-6
    else:
        # the mean is the library's own row terms averaged (fixed-order fp32 sum)
        assert abs(loss[0] - row.sum() / N) <= 1e-5 * np.abs(row).mean() + 1e-7


def run(x, t, w, grad_loss=1.0):
    xg, tg = x.cuda(), t.cuda()
    wg = None if w is None else w.cuda()
    got = fa.lsm_loss_fwd(xg, tg, wg)
    g = torch.tensor([grad_loss], dtype=torch.float32, device="cuda")
    fa.lsm_loss_bwd(xg, tg, wg, got[2], got[3], got[4], g)
    torch.cuda.synchronize()
    return got, xg


@pytest.mark.parametrize("N,V", [(1, 1), (3, 2), (5, 3), (7, 5), (16, 128), (33, 1000), (9, 1003),
                                 (4, 4097), (2, 32000)])
@pytest.mark.parametrize("masked", [False, True])
def test_loss_parity_small(N, V, masked):
    say(f"loss parity N={N} V={V} masked={masked}")
    g = torch.Generator().manual_seed(N * 7919 + V)
    x = torch.randn(N, V, generator=g) * 4
    u = torch.rand(N, V, generator=g) ** 8
    t = u / u.sum(dim=1, keepdim=True)
    w = (torch.rand(N, generator=g) > 0.3).float() if masked else None
    got, xg = run(x, t, w, grad_loss=0.75)
    check(x, t, w, xg, got, grad_loss=0.75)


def test_loss_parity_unnormalised_targets_and_weights():
    say("loss parity: targets not summing to 1, real-valued weights, wide logits")
    g = torch.Generator().manual_seed(11)
    N, V = 12, 777
    x = torch.randn(N, V, generator=g) * 20 - 5
    t = torch.rand(N, V, generator=g) * 0.01
    w = torch.rand(N, generator=g) * 3 - 1
    got, xg = run(x, t, w, grad_loss=-2.0)
    check(x, t, w, xg, got, grad_loss=-2.0)


def test_loss_strided_rows():
    say("loss parity: row strides above V")
    g = torch.Generator().manual_seed(12)
    N, V = 6, 250
    xb = torch.randn(N, 260, generator=g) * 4
    tb = torch.rand(N, 264, generator=g)
    x, t = xb[:, :V], tb[:, :V] / tb[:, :V].sum(dim=1, keepdim=True)
    xg, tg = xb.cuda()[:, :V], (tb[:, :V] / tb[:, :V].sum(dim=1, keepdim=True)).cuda()
    tgs = torch.zeros(N, 264, device="cuda")
    tgs[:, :V] = tg
    tgv = tgs[:, :V]
    got = fa.lsm_loss_fwd(xg, tgv, None)
    fa.lsm_loss_bwd(xg, tgv, None, got[2], got[3], got[4], torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    check(x, t, None, xg, got)
    # columns past V are untouched
    assert torch.equal(xb.cuda()[:, V:], xg.as_strided((N, 260), (260, 1))[:, V:])


def test_loss_rows_aligned_differently():
    # logits rows 1003 floats apart, target rows 1004: the two rows of a pair
    # sit at different offsets from a 16-byte boundary, so every element goes
    # one by one
    say("loss parity: logits and target rows aligned differently")
    g = torch.Generator().manual_seed(14)
    N, V = 7, 1003
    x = torch.randn(N, V, generator=g) * 4
    tb = torch.rand(N, 1004, generator=g)
    tb[:, :V] /= tb[:, :V].sum(dim=1, keepdim=True)
    xg = x.cuda()
    tg = tb.cuda()[:, :V]
    got = fa.lsm_loss_fwd(xg, tg, None)
    fa.lsm_loss_bwd(xg, tg, None, got[2], got[3], got[4], torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    check(x, tb[:, :V], None, xg, got)


def test_loss_deterministic_and_empty():
    say("loss: bitwise reruns, N = 0")
    x, t, w = W.make_loss_inputs(W.LossWorkload("t", 2, 300, 5000), seed=3)
    outs = []
    for _ in range(2):
        got, xg = run(x, t, w)
        outs.append([a.clone() for a in got] + [xg.clone()])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    e = torch.empty(0, 17, device="cuda")
    loss, row, m, d, ts = fa.lsm_loss_fwd(e, e.clone(), None)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and row.numel() == 0


def test_logsoftmax_loss_autograd_in_place():
    say("loss autograd: gradient written over the logits' storage")
    g = torch.Generator().manual_seed(13)
    N, V = 20, 3000
    x = torch.randn(N, V, generator=g) * 4
    u = torch.rand(N, V, generator=g) ** 8
    t = u / u.sum(dim=1, keepdim=True)
    w = (torch.arange(N) >= 3).float()
    leaf = x.cuda().requires_grad_(True)
    logits = leaf * 1.0          # an intermediate, as the LM head's output is
    loss = fa.logsoftmax_loss(logits, t.cuda(), w.cuda())
    (3.0 * loss).backward()
    torch.cuda.synchronize()
    ref_loss, *_ = lfwd(np64(x), np64(t), np64(w))
    assert abs(loss.item() - ref_loss) <= 1e-5 * max(1.0, abs(ref_loss))
    gref = lbwd(np64(x), np64(t), np64(w), grad_loss=3.0)
    # the gradient was written over the logits' own storage (no second
    # [N, V] buffer) and reached the leaf through the multiply
    assert np.abs(np64(logits) - gref).max() <= 1e-5 * np.abs(gref).max()
    assert np.abs(np64(leaf.grad) - gref).max() <= 1e-5 * np.abs(gref).max()


def test_loss_full_size_sampled_rows():
    # the page's largest configuration, in the benchmark's launch: every row
    # computed; every row term and the mean checked against the oracle (row
    # blocks of the fp64 oracle over the whole matrix), the gradient on
    # sampled rows
    w_ = W.LOSS_HEADLINE
    say(f"loss full size {w_.name}: N={w_.N} V={w_.V}")
    x, t, w = W.make_loss_inputs(w_, seed=1, device="cuda")
    x0 = x.clone()
    rows = np.unique(np.concatenate([[0, 1, w_.N // 2, w_.N - 1],
                                     np.random.default_rng(5).integers(0, w_.N, 28)]))
    xs, ts = x[rows].cpu(), t[rows].cpu()
    got = fa.lsm_loss_fwd(x, t, w)
    fa.lsm_loss_bwd(x, t, w, got[2], got[3], got[4], torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    gx = x  # the logits' storage now holds the gradient
    loss, row, m, d, tsum = got
    X, T, Wt = np64(xs), np64(ts), np64(w)[rows]
    _, rref, mref, dref, tref = lfwd(X, T, Wt)
    lse = mref + np.log(dref)
    scale = (np.abs(T) * (np.abs(X) + np.abs(lse)[:, None])).sum(axis=1)
    assert np.array_equal(np64(m)[rows], mref)
    assert np.abs(np64(d)[rows] / dref - 1).max() <= 1e-5
    assert np.abs(np64(tsum)[rows] - tref).max() <= 1e-5
    assert np.all(np.abs(np64(row)[rows] - rref) <= 2e-5 * scale + 1e-6)
    gref = lbwd(X, T, Wt) * len(rows) / w_.N
    G = np64(gx[rows])
    assert np.all(np.abs(G - gref).max(axis=1) <= 1e-5 * np.abs(gref).max(axis=1) + 1e-12)
    # every row term and the mean against the oracle, 1024 rows at a time
    r = np64(row)
    ref_rows = np.empty(w_.N)
    bound = np.empty(w_.N)
    Wall = np64(w)
    for r0 in range(0, w_.N, 1024):
        sl = slice(r0, min(w_.N, r0 + 1024))
        Xb, Tb = np64(x0[sl]), np64(t[sl])
        _, rb, mb, db, _ = lfwd(Xb, Tb, Wall[sl])
        ref_rows[sl] = rb
        bound[sl] = 2e-5 * (np.abs(Tb) * (np.abs(Xb) + np.abs(mb + np.log(db))[:, None])).sum(axis=1) + 1e-6
    assert np.all(np.abs(r - ref_rows) <= bound), "row terms"
    mean_ref = ref_rows.sum() / w_.N
    err = abs(np64(loss)[0] - mean_ref)
    say(f"loss full size: mean {np64(loss)[0]:.8f} oracle {mean_ref:.8f} |err| {err:.2e}")
    assert err <= bound.sum() / w_.N
