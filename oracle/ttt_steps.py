"""Step-by-step EAGLE3 training-time-test (TTT) attention, fp64 torch on CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  This is a second,
independent formulation of the TTT mask, used to pin the predicate oracle in
``oracle/attention.py``; it never looks at a mask matrix.

Source: "Flex Attention and Triton, Supporting Long Context Training in
SpecForge", section *EAGLE3 Training*, the naive TTT attention: scores of the
queries against the step-0 keys form a causal block; for every earlier draft
step s >= 1 the query at position i takes one more score, the dot product with
that step's cached key at the same position i; all scores go through one
joint softmax; the output is the block's weights times the step-0 values plus,
for each step s, the weight of its extra column times that step's value at
position i.

Readings where the page is unclear: the extra columns exist for cache steps
1..t only (step 0 is the causal block); ``qi`` in the page's loop is the query
rows themselves; a padding length kv_valid removes key positions >= kv_valid
of every step; an optional causal shift applies to the step-0 block only, as
the flex mask applies it to its causal part only.

Written with torch ops so a test can differentiate it with fp64 autograd.
"""
import torch


def ttt_stepwise_forward(q, k_steps, v_steps, shift=0, kv_valid=None,
                         scale=None):
    """O [B,Hq,L,D] and LSE [B,Hq,L] for the TTT call at step t.

    q: [B,Hq,L,D]; k_steps, v_steps: lists of t+1 tensors [B,Hkv,L,D] (the
    cached keys/values of steps 0..t).  float64 torch tensors.
    """
    B, Hq, L, D = q.shape
    Hkv = k_steps[0].shape[1]
    G = Hq // Hkv
    s = 1.0 / D ** 0.5 if scale is None or scale <= 0 else float(scale)
    n_steps = len(k_steps)
    pos = torch.arange(L)
    outs, lses = [], []
    for b in range(B):
        n_valid = L if kv_valid is None else int(kv_valid[b])
        block_ok = (pos[:, None] - shift >= pos[None, :]) & (pos[None, :] < n_valid)
        col_ok = pos < n_valid                       # key position i of step s
        o_b, l_b = [], []
        for h in range(Hq):
            g = h // G
            qh = q[b, h]
            block = s * (qh @ k_steps[0][b, g].T)                 # [L, L]
            cols = [s * (qh * k_steps[st][b, g]).sum(-1)          # [L]
                    for st in range(1, n_steps)]
            scores = torch.cat([block] + [c[:, None] for c in cols], dim=1)
            ok = torch.cat([block_ok] + [col_ok[:, None]] * (n_steps - 1), dim=1)
            nonempty = ok.any(dim=1)
            # masked entries become -inf; rows with nothing allowed are zeroed
            safe = torch.where(ok, scores, torch.full_like(scores, -torch.inf))
            safe = torch.where(nonempty[:, None], safe, torch.zeros_like(safe))
            lse = torch.logsumexp(safe, dim=1)
            w = torch.exp(safe - lse[:, None])
            w = torch.where(nonempty[:, None] & ok, w, torch.zeros_like(w))
            out = w[:, :L] @ v_steps[0][b, g]
            for st in range(1, n_steps):
                out = out + w[:, L + st - 1, None] * v_steps[st][b, g]
            o_b.append(out)
            l_b.append(torch.where(nonempty, lse, torch.zeros_like(lse)))
        outs.append(torch.stack(o_b))
        lses.append(torch.stack(l_b))
    return torch.stack(outs), torch.stack(lses)
