"""fp64 soft-target log-softmax loss and its gradient with respect to the logits.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "Flex Attention and Triton, Supporting Long Context Training in
SpecForge", section *In-place Gradient Calculation*.  Per TTT step, EAGLE3
training takes the log-softmax of the draft model's logits over the
vocabulary, weights it by the target model's (soft) probabilities and by the
position mask of each row, sums over the vocabulary, negates, and averages
over the (batch, position) rows.  The page's fused kernel keeps, per row, the
max m of the logits and the normaliser d = sum_v exp(x_v - m), and its
backward writes the gradient into the logits' own buffer; the gradient of
the row term is -(t_v * g - softmax_v * sum_u t_u * g) for the row's upstream
gradient g.

Everything here is that definition written out in float64 on the whole
[N, V] matrix, nothing fused:

    m_i      = max_v x_iv
    d_i      = sum_v exp(x_iv - m_i)
    logp_iv  = x_iv - m_i - ln d_i
    row_i    = -w_i * sum_v t_iv * logp_iv
    loss     = (1/N) * sum_i row_i
    dloss/dx_iv * g = g * w_i / N * (exp(logp_iv) * sum_u t_iu - t_iv)

Readings taken where the page is silent:
  * the mean runs over all N = B * T rows, masked rows included (the page
    applies the mask inside the vocabulary sum and then takes ``.mean()``);
  * the position mask is a per-row weight w_i (0 or 1 on the page, any real
    value here);
  * the targets need not sum to 1: the gradient keeps the factor sum_u t_iu
    that the page's kernel computes as its first backward pass;
  * g is the upstream gradient of the scalar (mean) loss.

Pinned in tests/test_oracle_pins_loss.py against torch's cross_entropy on
one-hot targets (a different library routine), a two-class closed form,
uniform-logit closed forms, invariants and central finite differences.
"""
import numpy as np


def _rows(x):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("expected [N, V]")
    return x


def logsoftmax_loss_forward(logits, target, mask=None):
    """Returns (loss, row, m, d, tsum): the mean loss (float), the per-row
    terms row_i = -w_i sum_v t_iv logp_iv, the row max m, the normaliser d
    and the row sums of the target, all float64."""
    x, t = _rows(logits), _rows(target)
    N = x.shape[0]
    w = np.ones(N) if mask is None else np.asarray(mask, dtype=np.float64).reshape(N)
    m = x.max(axis=1) if x.shape[1] else np.zeros(N)
    d = np.exp(x - m[:, None]).sum(axis=1)
    logp = x - m[:, None] - np.log(d)[:, None]
    row = -w * (t * logp).sum(axis=1)
    loss = row.sum() / N if N else 0.0
    return loss, row, m, d, t.sum(axis=1)


def logsoftmax_loss_backward(logits, target, mask=None, grad_loss=1.0):
    """Gradient of grad_loss * loss with respect to the logits, [N, V] float64."""
    x, t = _rows(logits), _rows(target)
    N = x.shape[0]
    w = np.ones(N) if mask is None else np.asarray(mask, dtype=np.float64).reshape(N)
    m = x.max(axis=1)
    d = np.exp(x - m[:, None]).sum(axis=1)
    p = np.exp(x - m[:, None]) / d[:, None]
    coef = float(grad_loss) * w / N
    return coef[:, None] * (p * t.sum(axis=1)[:, None] - t)
