"""Pins of the fp64 log-softmax loss oracle (oracle/loss.py) to things other
than itself: torch's cross_entropy on one-hot targets (a different library
routine), a two-class closed form, uniform-logit closed forms, invariants
and central finite differences.

The loss is the EAGLE3 soft-target loss of "Flex Attention and Triton,
Supporting Long Context Training in SpecForge", section *In-place Gradient
Calculation*.
"""
import math

import numpy as np
import pytest
import torch

from oracle import logsoftmax_loss_forward as lfwd, logsoftmax_loss_backward as lbwd


def rnd(seed, N, V, scale=3.0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((N, V)) * scale
    t = r.random((N, V))
    t /= t.sum(axis=1, keepdims=True)
    return x, t


@pytest.mark.parametrize("N,V", [(1, 2), (5, 7), (16, 100)])
def test_one_hot_targets_equal_torch_cross_entropy(N, V):
    # One-hot targets and no mask: the loss is the textbook cross entropy,
    # mean over rows, and the gradient is its autograd gradient.
    r = np.random.default_rng(N * 1000 + V)
    x = r.standard_normal((N, V)) * 4
    cls = r.integers(0, V, size=N)
    t = np.zeros((N, V))
    t[np.arange(N), cls] = 1.0
    loss, row, m, d, tsum = lfwd(x, t)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    ref = torch.nn.functional.cross_entropy(xt, torch.tensor(cls), reduction="mean")
    ref.backward()
    assert abs(loss - ref.item()) <= 1e-12 * max(1.0, abs(ref.item()))
    g = lbwd(x, t, grad_loss=1.0)
    assert np.abs(g - xt.grad.numpy()).max() <= 1e-13
    # per-row terms are the per-row cross entropies
    rows = torch.nn.functional.cross_entropy(xt.detach(), torch.tensor(cls), reduction="none").numpy()
    assert np.abs(row - rows).max() <= 1e-12
    assert np.allclose(tsum, 1.0)


def test_two_class_closed_form():
    # V = 2, logits (a, b), targets (p, q): the loss is -(p ln s(a-b) + q ln s(b-a))
    # with s the logistic function; the gradient is (s(a-b) (p+q) - p, s(b-a) (p+q) - q).
    a, b, p, q = 1.25, -0.5, 0.3, 0.9
    s = lambda z: 1.0 / (1.0 + math.exp(-z))
    loss, *_ = lfwd([[a, b]], [[p, q]])
    assert abs(loss - (-(p * math.log(s(a - b)) + q * math.log(s(b - a))))) <= 1e-15
    g = lbwd([[a, b]], [[p, q]], grad_loss=2.0)
    ref = 2.0 * np.array([s(a - b) * (p + q) - p, s(b - a) * (p + q) - q])
    assert np.abs(g[0] - ref).max() <= 1e-15


def test_uniform_logits_closed_form():
    # every logit of a row equal to c: logp = -ln V, so row_i = w_i ln V sum_v t_iv,
    # m = c, d = V, and the gradient is g w_i / N (sum_u t_u / V - t_v)
    N, V = 4, 9
    r = np.random.default_rng(3)
    c = r.standard_normal(N)
    x = np.repeat(c[:, None], V, axis=1)
    t = r.random((N, V))
    w = np.array([1.0, 0.0, 2.5, 1.0])
    loss, row, m, d, tsum = lfwd(x, t, w)
    assert np.allclose(row, w * math.log(V) * t.sum(axis=1), rtol=0, atol=1e-14)
    assert np.allclose(m, c, rtol=0, atol=0) and np.allclose(d, V, rtol=0, atol=1e-13)
    assert abs(loss - row.sum() / N) <= 1e-15
    g = lbwd(x, t, w, grad_loss=0.5)
    ref = 0.5 * w[:, None] / N * (t.sum(axis=1, keepdims=True) / V - t)
    assert np.abs(g - ref).max() <= 1e-15


def test_row_shift_invariance_and_zero_gradient_sum():
    # adding a constant to a row's logits changes neither its loss nor its
    # gradient; the gradient of each row sums to 0 (softmax sums to 1)
    x, t = rnd(4, 6, 50)
    w = np.array([1, 0, 1, 1, 0.5, 1.0])
    loss, row, m, d, _ = lfwd(x, t, w)
    sh = np.arange(6)[:, None] * 7.5 - 10
    loss2, row2, m2, d2, _ = lfwd(x + sh, t, w)
    assert np.abs(row - row2).max() <= 1e-12 and abs(loss - loss2) <= 1e-12
    assert np.allclose(m2, m + sh[:, 0]) and np.allclose(d2, d)
    g, g2 = lbwd(x, t, w), lbwd(x + sh, t, w)
    assert np.abs(g - g2).max() <= 1e-15
    assert np.abs(g.sum(axis=1)).max() <= 1e-15


def test_masked_rows_contribute_nothing():
    x, t = rnd(5, 4, 30)
    w = np.array([0.0, 1.0, 0.0, 1.0])
    loss, row, *_ = lfwd(x, t, w)
    assert row[0] == 0.0 and row[2] == 0.0
    g = lbwd(x, t, w)
    assert np.all(g[0] == 0.0) and np.all(g[2] == 0.0)
    # the mean still divides by all rows
    _, row_all, *_ = lfwd(x, t)
    assert abs(loss - (row_all[1] + row_all[3]) / 4) <= 1e-14


def test_linear_in_target_scale():
    # unnormalised targets: the loss and the gradient are linear in t
    x, t = rnd(6, 3, 20)
    l1, *_ = lfwd(x, t)
    l3, *_ = lfwd(x, 3.0 * t)
    assert abs(l3 - 3.0 * l1) <= 1e-13
    assert np.abs(lbwd(x, 3.0 * t) - 3.0 * lbwd(x, t)).max() <= 1e-15


@pytest.mark.parametrize("seed", [0, 1])
def test_gradient_equals_central_finite_differences(seed):
    N, V = 3, 11
    x, t = rnd(seed, N, V, scale=2.0)
    t *= np.array([1.0, 0.7, 1.3])[:, None]          # targets not summing to 1
    w = np.array([1.0, 0.5, 1.0])
    gl = 1.7
    g = lbwd(x, t, w, grad_loss=gl)
    h = 1e-6
    num = np.zeros_like(x)
    for i in range(N):
        for v in range(V):
            xp, xm = x.copy(), x.copy()
            xp[i, v] += h
            xm[i, v] -= h
            num[i, v] = gl * (lfwd(xp, t, w)[0] - lfwd(xm, t, w)[0]) / (2 * h)
    assert np.abs(num).max() > 1e-3
    assert np.abs(g - num).max() <= 1e-8
