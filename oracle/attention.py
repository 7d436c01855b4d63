"""fp64 materialised attention: forward (O, LSE) and analytic backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources, by page and section:

* "Flex Attention and Triton, Supporting Long Context Training in SpecForge",
  section *EAGLE3 Training*: attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V,
  with the softmax taken in fp32 or better.
* Same page, section *Flex Attention*: the EAGLE3 mask is the OR of a causal
  part (query index minus a shift at least the key index, key index below the
  batch's sequence length) and a suffix part (key index at least Q_LEN, key
  index modulo Q_LEN below the sequence length, and key minus query index a
  multiple of Q_LEN).  The mask does not depend on the head (H=1 broadcast) and
  K/V heads are shared by groups of query heads (enable_gqa).
* "Flash-attention training (the fused backward) - adoption playbook",
  section *1. What exists*: the forward's saved state is O plus the per-row
  logsumexp LSE; the backward produces dQ, dK, dV.  Section *6. Trap list*,
  item 9: a query row with no allowed key has O = 0 and LSE = 0; item 8: a key
  column no query may attend gets an exactly-zero gradient.
* "CS336 - LLM Systems", *Flash Attention (Triton)* / *How it works*: the
  fused kernel returns the same result as the explicit
  Q K^T -> softmax -> P V chain; only memory traffic changes.
* The playbook, section *4. Measurement discipline*: the diffusion trainer's
  attention geometries include windowed self-attention besides full
  self-attention and cross-attention.  The page does not define the window;
  WINDOW here is a band of key positions around the query position (see
  ``allowed``).
* The playbook, section *3. Per-trainer porting checklist*: the fused ops
  take an additive mask, added to the scores before the softmax and
  broadcast where it has fewer dimensions.  ``bias`` here is its per-batch,
  per-key form [B, Skv]: bias[b, j] is added to the scaled score of every
  query row and head of batch entry b with key j, on top of the mask kind
  (a key with bias -inf is dropped for that batch entry).  It is an input
  only: the page's backward produces dQ, dK and dV, nothing for the mask.

Readings taken where the pages are silent:
  * scale defaults to 1/sqrt(D);
  * LSE is the natural-log logsumexp of the *scaled* scores;
  * CAUSAL with Sq != Skv is top-left aligned: key j allowed iff j <= i - shift;
  * kv_valid[b] masks keys only, every query row is computed;
  * GQA maps query head h to key/value head h // (Hq / Hkv);
  * WINDOW (left, right): key j allowed iff
    i - shift - left <= j <= i - shift + right (and j below kv_valid), so
    (left, 0) is a causal sliding window of left + 1 keys and (w, w) a
    symmetric band;
  * the additive mask is taken in its per-(batch, key) form, which keeps the
    path linear in S (a dense [Sq, Skv] mask is an S x S tensor in memory);
    its values are real numbers or -inf (the page's F16 mask values are
    among them); LSE includes it.

With a bias the scores are  S = scale * Q K^T + bias[b]  (the bias row
broadcast over query rows and heads); everything below uses those scores.

The backward is the gradient of  L = sum(O * dO)  (dO is the upstream
gradient), derived from the softmax Jacobian:
    dV = P^T dO,  dP = dO V^T,  Delta_i = sum_j P_ij dP_ij,
    dS = P * (dP - Delta),  dQ = scale * dS K,  dK = scale * dS^T Q.
"""
import numpy as np

FULL, CAUSAL, TTT, WINDOW = 0, 1, 2, 3

# Rows of S materialised at a time; only bounds RAM, never splits a row.
_ROW_BLOCK = 1024


def allowed(kind, Sq, Skv, shift=0, kv_valid=None, rows=None, window=None):
    """Boolean [len(rows), Skv] matrix: may query i attend key j?

    A literal transcription of the masks on the SpecForge page (*Flex
    Attention* section): FULL is the padding mask alone, CAUSAL is the
    ``causal_mask`` function, TTT is ``or_masks(causal_mask, suffix_mask)``
    with Q_LEN = Sq.  ``kv_valid`` plays the role of ``seq_lengths[b]``.
    WINDOW (``window`` = (left, right)) is the band
    i - shift - left <= j <= i - shift + right with the padding mask.
    """
    i = (np.arange(Sq) if rows is None else np.asarray(rows))[:, None]
    j = np.arange(Skv)[None, :]
    n_valid = Skv if kv_valid is None else int(kv_valid)
    padding = j < n_valid
    if kind == FULL:
        return np.broadcast_to(padding, (i.shape[0], Skv)).copy()
    causal = (i - shift >= j) & padding
    if kind == CAUSAL:
        return causal
    if kind == TTT:
        q_len = Sq
        suffix = (j >= q_len) & ((j % q_len) < n_valid) & (((j - i) % q_len) == 0)
        return causal | suffix
    if kind == WINDOW:
        left, right = window
        return (j >= i - shift - left) & (j <= i - shift + right) & padding
    raise ValueError(f"unknown mask kind {kind}")


def allowed_pair_count(kind, Sq, Skv, shift=0, kv_valid=None, window=None):
    """Number of allowed (i, j) pairs for one (batch, head): the unit in which
    attention work is counted (4 D flop per pair forward, 10 D backward)."""
    total = 0
    for r0 in range(0, Sq, 4096):
        rows = np.arange(r0, min(Sq, r0 + 4096))
        total += int(allowed(kind, Sq, Skv, shift, kv_valid, rows, window).sum())
    return total


def _kv_valid_list(B, Skv, kv_valid):
    if kv_valid is None:
        return [Skv] * B
    return [int(x) for x in np.asarray(kv_valid).reshape(-1)]


def _bias_rows(B, Skv, bias):
    """The per-batch key bias as a float64 [B, Skv] array (zeros if None)."""
    if bias is None:
        return np.zeros((B, Skv))
    b = np.asarray(bias, dtype=np.float64)
    assert b.shape == (B, Skv), f"bias must be [B, Skv], got {b.shape}"
    return b


def _check_shapes(q, k, v):
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    assert v.shape == k.shape and Bk == B and Dk == D
    assert Hq % Hkv == 0, "GQA needs Hq to be a multiple of Hkv"
    return B, Hq, Hkv, Sq, Skv, D


def _row_softmax(S_masked):
    """Softmax of masked score rows, plus the per-row natural logsumexp.

    Rows with no allowed key give P = 0 and LSE = 0 (playbook trap 9).
    """
    nonempty = np.isfinite(S_masked).any(axis=1)
    m = np.where(nonempty, S_masked.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(S_masked - m[:, None])          # exp(-inf) = 0 for masked entries
    e[~nonempty] = 0.0
    z = e.sum(axis=1)
    lse = np.where(nonempty, m + np.log(np.where(nonempty, z, 1.0)), 0.0)
    P = np.where(nonempty[:, None], e / np.where(nonempty, z, 1.0)[:, None], 0.0)
    return P, lse


def _row_blocks(Sq, rows):
    """Query-row blocks to materialise: all rows, or the sampled range."""
    lo, hi = (0, Sq) if rows is None else (int(rows[0]), int(rows[1]))
    for r0 in range(lo, hi, _ROW_BLOCK):
        yield np.arange(r0, min(hi, r0 + _ROW_BLOCK))


def attention_forward(q, k, v, kind=FULL, shift=0, kv_valid=None, scale=None,
                      heads=None, rows=None, window=None, bias=None):
    """O [B,Hq,Sq,D] and LSE [B,Hq,Sq] in float64.

    ``heads`` (a list of query heads) and ``rows`` (a half-open range
    (lo, hi) of query rows) optionally restrict the work; outputs outside the
    selection are left as NaN.  Used to check or time a sample of a large
    configuration; every computed row is still complete over all keys.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, Hq, Hkv, Sq, Skv, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    s = 1.0 / np.sqrt(D) if scale is None or scale <= 0 else float(scale)
    kvv = _kv_valid_list(B, Skv, kv_valid)
    bias = _bias_rows(B, Skv, bias)
    hs = range(Hq) if heads is None else heads
    O = np.full(q.shape, np.nan)
    LSE = np.full((B, Hq, Sq), np.nan)
    for b in range(B):
        for rb in _row_blocks(Sq, rows):
            A = allowed(kind, Sq, Skv, shift, kvv[b], rb, window)
            for h in hs:
                g = h // G
                S = s * (q[b, h, rb] @ k[b, g].T) + bias[b][None, :]
                P, lse = _row_softmax(np.where(A, S, -np.inf))
                O[b, h, rb] = P @ v[b, g]
                LSE[b, h, rb] = lse
    return O, LSE


def attention_backward(q, k, v, do, kind=FULL, shift=0, kv_valid=None,
                       scale=None, heads=None, rows=None, window=None, bias=None):
    """dQ, dK, dV (float64) of L = sum(O * dO), plus Delta [B,Hq,Sq].

    P is rebuilt from the scores, exactly as the definition states; dK and dV
    of a key/value head sum the contributions of every query head in its
    group.  With ``heads`` / ``rows`` only the selected query rows contribute
    (to dK/dV as well), and the other dQ rows are NaN.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, Hkv, Sq, Skv, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    s = 1.0 / np.sqrt(D) if scale is None or scale <= 0 else float(scale)
    kvv = _kv_valid_list(B, Skv, kv_valid)
    bias = _bias_rows(B, Skv, bias)
    hs = range(Hq) if heads is None else heads
    dQ = np.full(q.shape, np.nan)
    dK = np.zeros(k.shape)
    dV = np.zeros(v.shape)
    Delta = np.full((B, Hq, Sq), np.nan)
    for b in range(B):
        for rb in _row_blocks(Sq, rows):
            A = allowed(kind, Sq, Skv, shift, kvv[b], rb, window)
            for h in hs:
                g = h // G
                S = s * (q[b, h, rb] @ k[b, g].T) + bias[b][None, :]
                P, _ = _row_softmax(np.where(A, S, -np.inf))
                dO = do[b, h, rb]
                dV[b, g] += P.T @ dO
                dP = dO @ v[b, g].T
                delta = (P * dP).sum(axis=1)
                dS = P * (dP - delta[:, None])
                dQ[b, h, rb] = s * (dS @ k[b, g])
                dK[b, g] += s * (dS.T @ q[b, h, rb])
                Delta[b, h, rb] = delta
    return dQ, dK, dV, Delta


def attention_key_grads(q, k, v, do, keys, kind=FULL, shift=0, kv_valid=None, scale=None,
                        window=None, bias=None):
    """dK, dV (float64) of the keys [keys[0], keys[1]) only, over every query
    row and every head of each group: [B, Hkv, k1 - k0, D] each.

    The gradient of one key needs every query row that may attend it, and of
    those rows the logsumexp and output over their complete key sets.  So:
    the rows that may attend some key of the range are found from the mask;
    their LSE and O come from ``attention_forward`` (complete rows); then, as
    the CS336 page's backward does, P of the range's keys is recomputed from
    the scores and the saved logsumexp, P_ij = exp(s q_i.k_j - LSE_i) on
    allowed pairs (0 elsewhere), and with dP_ij = dO_i.v_j,
    Delta_i = sum_d dO_id O_id (which equals sum_j P_ij dP_ij, because
    O_i = sum_j P_ij v_j) and dS = P (dP - Delta):
        dV_j = sum_i P_ij dO_i,    dK_j = s sum_i dS_ij q_i,
    summed over the query heads of the key's group.  The same values as
    ``attention_backward``'s dK, dV on those keys, without materialising the
    other keys' gradients.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, Hkv, Sq, Skv, D = _check_shapes(q, k, v)
    G = Hq // Hkv
    s = 1.0 / np.sqrt(D) if scale is None or scale <= 0 else float(scale)
    kvv = _kv_valid_list(B, Skv, kv_valid)
    bias = _bias_rows(B, Skv, bias)
    k0, k1 = int(keys[0]), int(keys[1])
    dK = np.zeros((B, Hkv, k1 - k0, D))
    dV = np.zeros((B, Hkv, k1 - k0, D))
    for b in range(B):
        # rows that may attend a key of the range (scanned in row blocks)
        att = np.zeros(Sq, bool)
        for rb in _row_blocks(Sq, None):
            att[rb] = allowed(kind, Sq, Skv, shift, kvv[b], rb, window)[:, k0:k1].any(1)
        rows = np.nonzero(att)[0]
        if len(rows) == 0:
            continue
        lo, hi = int(rows[0]), int(rows[-1]) + 1
        for g in range(Hkv):
            heads = list(range(g * G, (g + 1) * G))
            O, LSE = attention_forward(q[b:b + 1], k[b:b + 1], v[b:b + 1], kind, shift,
                                       [kvv[b]], s, heads=heads, rows=(lo, hi), window=window,
                                       bias=bias[b:b + 1])
            for rb in _row_blocks(Sq, (lo, hi)):
                A = allowed(kind, Sq, Skv, shift, kvv[b], rb, window)[:, k0:k1]
                for h in heads:
                    S = s * (q[b, h, rb] @ k[b, g, k0:k1].T) + bias[b, k0:k1][None, :]
                    P = np.where(A, np.exp(np.where(A, S, 0.0) - LSE[0, h, rb][:, None]), 0.0)
                    dO = do[b, h, rb]
                    dP = dO @ v[b, g, k0:k1].T
                    delta = (dO * O[0, h, rb]).sum(axis=1)
                    dS = P * (dP - delta[:, None])
                    dV[b, g] += P.T @ dO
                    dK[b, g] += s * (dS.T @ q[b, h, rb])
    return dK, dV


def attention_ref(q, k, v, do, kind=FULL, shift=0, kv_valid=None, scale=None,
                  heads=None, rows=None, window=None, bias=None):
    """Forward and backward together: dict with O, LSE, dQ, dK, dV, Delta."""
    O, LSE = attention_forward(q, k, v, kind, shift, kv_valid, scale, heads, rows, window, bias)
    dQ, dK, dV, Delta = attention_backward(q, k, v, do, kind, shift, kv_valid,
                                           scale, heads, rows, window, bias)
    return dict(O=O, LSE=LSE, dQ=dQ, dK=dK, dV=dV, Delta=Delta)
