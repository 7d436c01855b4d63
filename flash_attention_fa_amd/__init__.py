"""MI355X (gfx950) fused training attention: forward, backward, autograd.

Thin Python binding over ``libfa.so`` (include/fa.h).  Every step of the
computation runs in the library's HIP kernels; PyTorch only provides device
memory and the current stream.  The functions mirror the C entry points:

    fa_fwd(q, k, v, ...)                     -> (o, lse)
    fa_fwd_noalloc(q, k, v, ...)             -> (o, lse), workspace from the library's static array
    fa_fwd_workspace_bytes(q, k, ...)        -> int
    fa_bwd(q, k, v, o, lse, dout, ...)       -> (dq, dk, dv)
    fa_bwd_stage(stage, q, k, v, ..., dq, dk, dv, workspace)   (one stage of fa_bwd)
    fa_bwd_workspace_bytes(q, k, ...)        -> int
    fa_last_error()                          -> str

and ``attention(q, k, v, ...)`` is a drop-in ``torch.autograd.Function``
that saves (O, LSE) for the backward.

Tensors are logical [B, H, S, D] (any strides with unit stride in D): q is
[B, Hq, Sq, D], k and v are [B, Hkv, Skv, D] with Hq a multiple of Hkv.
Mask kinds: ``FULL``, ``CAUSAL`` (key j <= query i - causal_shift),
``TTT`` (EAGLE3 training-time test: Skv = n * Sq, causal over the step-0 keys
plus the key at the query's own position in each later step) and ``WINDOW``
(``window=(left, right)``: i - causal_shift - left <= j <= i - causal_shift +
right).  ``kv_valid`` is an optional int32 device tensor [B] of valid key
counts.  ``key_bias`` is an optional float32 device tensor [B, Skv] (unit key
stride; a stride of 0 over B shares one row) added to the scaled scores of
every query row and head: an additive mask in per-key form, -inf drops a key.
It receives no gradient.
"""
import torch

from . import _lib
from ._lib import (FAError, FA_BF16, FA_F32, FA_MASK_FULL, FA_MASK_CAUSAL,  # noqa: F401
                   FA_MASK_TTT, FA_MASK_WINDOW, FA_BWD_DELTA, FA_BWD_DKDV, FA_BWD_DQ)

FULL, CAUSAL, TTT, WINDOW = FA_MASK_FULL, FA_MASK_CAUSAL, FA_MASK_TTT, FA_MASK_WINDOW

__all__ = ["fa_fwd", "fa_fwd_noalloc", "fa_fwd_workspace_bytes", "fa_bwd", "fa_bwd_stage", "fa_bwd_workspace_bytes",
           "fa_last_error", "FA_BWD_DELTA", "FA_BWD_DKDV", "FA_BWD_DQ",
           "attention", "FAError", "FULL", "CAUSAL", "TTT", "WINDOW",
           "lsm_loss_fwd", "lsm_loss_bwd", "logsoftmax_loss"]


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise FAError(_lib.FA_ERR_UNSUPPORTED, f"dtype {t.dtype} (expected bfloat16 or float32)")


def _tensor(t):
    if t.dim() != 4:
        raise FAError(_lib.FA_ERR_INVALID_ARG, f"expected a 4-d [B, H, S, D] tensor, got {tuple(t.shape)}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise FAError(_lib.FA_ERR_INVALID_ARG, "the D dimension must have unit stride")
    return _lib.fa_tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _mask(kind, causal_shift, kv_valid, window=None, frozen_keys=0, key_bias=None, shape=None):
    ptr = None
    bias_ptr, bias_sb = None, 0
    if key_bias is not None:
        if key_bias.dtype != torch.float32 or key_bias.dim() != 2:
            raise FAError(_lib.FA_ERR_INVALID_ARG, "key_bias must be a 2-d float32 tensor [B, Skv]")
        if shape is not None and tuple(key_bias.shape) != shape:
            raise FAError(_lib.FA_ERR_INVALID_ARG, f"key_bias has shape {tuple(key_bias.shape)}, expected {shape}")
        if key_bias.shape[1] > 1 and key_bias.stride(1) != 1:
            raise FAError(_lib.FA_ERR_INVALID_ARG, "key_bias needs unit stride over keys")
        bias_ptr = key_bias.data_ptr()
        bias_sb = key_bias.stride(0) if key_bias.shape[0] > 1 else 0
    if kv_valid is not None:
        if kv_valid.dtype != torch.int32 or not kv_valid.is_contiguous():
            raise FAError(_lib.FA_ERR_INVALID_ARG, "kv_valid must be a contiguous int32 tensor")
        ptr = kv_valid.data_ptr()
    if int(kind) == WINDOW and window is None:
        raise FAError(_lib.FA_ERR_INVALID_ARG, "mask_kind WINDOW needs window=(left, right)")
    left, right = (0, 0) if window is None else (int(window[0]), int(window[1]))
    return _lib.fa_mask_desc(int(kind), int(causal_shift), ptr, left, right, int(frozen_keys),
                             bias_ptr, int(bias_sb))


def _bias_shape(q, k):
    return (int(q.shape[0]), int(k.shape[2]))


def _stream(t, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _scratch(nbytes, device, stream):
    """A workspace the binding allocates for one call.  It is freed when the
    call returns, while the kernels may still be running on ``stream``: the
    caching allocator must not hand its memory out again before that stream
    has finished with it (record_stream).  For a raw stream handle that
    cannot be recorded, the caller has to pass a workspace."""
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if stream is not None:
        if not isinstance(stream, torch.cuda.Stream):
            raise FAError(_lib.FA_ERR_INVALID_ARG,
                          "with a raw stream handle, pass workspace= (the binding cannot keep "
                          "its own scratch alive until that stream is done with it)")
        ws.record_stream(stream)
    return ws


def _shape(q, k):
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    return int(B), int(Hq), int(Hkv), int(Sq), int(Skv), int(D)


def _fwd_shape_args(q, k):
    B, Hq, Hkv, Sq, Skv, D = _shape(q, k)
    a = _lib.fa_fwd_args()
    a.dtype = _dtype_code(q)
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = B, Hq, Hkv, Sq, Skv, D
    return a


def fa_fwd_workspace_bytes(q, k, *, key_bias=None):
    """Scratch bytes fa_fwd needs for these shapes (bf16: a transposed V, and
    with a key bias a scaled copy of it; linear in Skv)."""
    a = _fwd_shape_args(q, k)
    a.mask = _mask(FULL, 0, None, None, 0, key_bias, _bias_shape(q, k))
    return int(_lib.lib().fa_fwd_workspace_bytes(a))


def fa_fwd(q, k, v, *, mask_kind=FULL, causal_shift=0, kv_valid=None, window=None, scale=None,
           out=None, lse=None, workspace=None, stream=None, frozen_keys=0, key_bias=None):
    """Forward attention.  Returns (O [B,Hq,Sq,D] in q's dtype, LSE [B,Hq,Sq] fp32).

    ``workspace`` (uint8 device tensor of at least ``fa_fwd_workspace_bytes``
    bytes) is allocated when not given."""
    B, Hq, Hkv, Sq, Skv, D = _shape(q, k)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    a = _fwd_shape_args(q, k)
    a.scale = 0.0 if scale is None else float(scale)
    a.q, a.k, a.v, a.o = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    a.lse = lse.data_ptr()
    a.mask = _mask(mask_kind, causal_shift, kv_valid, window, frozen_keys, key_bias, _bias_shape(q, k))
    for t in (k, v, out):
        if t.dtype != q.dtype:
            raise FAError(_lib.FA_ERR_INVALID_ARG, "q, k, v and out must share one dtype")
    need = int(_lib.lib().fa_fwd_workspace_bytes(a))
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    _lib.check(_lib.lib().fa_fwd(a, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _stream(q, stream)))
    return out, lse


def fa_fwd_noalloc(q, k, v, *, mask_kind=FULL, causal_shift=0, kv_valid=None, window=None, scale=None,
                   out=None, lse=None, stream=None, frozen_keys=0, key_bias=None):
    """fa_fwd without a workspace argument: the library's static device
    scratch holds the transposed V (for callers that cannot allocate, e.g.
    under graph capture; pass ``out`` and ``lse`` there, since allocating
    them here would defeat the purpose).  Same results as fa_fwd, bitwise.
    Calls that overlap in time on one device share the scratch and race."""
    B, Hq, Hkv, Sq, Skv, D = _shape(q, k)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    a = _fwd_shape_args(q, k)
    a.scale = 0.0 if scale is None else float(scale)
    a.q, a.k, a.v, a.o = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    a.lse = lse.data_ptr()
    a.mask = _mask(mask_kind, causal_shift, kv_valid, window, frozen_keys, key_bias, _bias_shape(q, k))
    for t in (k, v, out):
        if t.dtype != q.dtype:
            raise FAError(_lib.FA_ERR_INVALID_ARG, "q, k, v and out must share one dtype")
    _lib.check(_lib.lib().fa_fwd_noalloc(a, _stream(q, stream)))
    return out, lse


def _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, mask_kind, causal_shift, kv_valid, scale, window=None,
              frozen_keys=0, key_bias=None):
    B, Hq, Hkv, Sq, Skv, D = _shape(q, k)
    a = _lib.fa_bwd_args()
    a.dtype = _dtype_code(q)
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = B, Hq, Hkv, Sq, Skv, D
    a.scale = 0.0 if scale is None else float(scale)
    a.q, a.k, a.v, a.o, a.dout = (_tensor(t) for t in (q, k, v, o, dout))
    a.lse = None if lse is None else lse.data_ptr()
    if dq is not None:
        a.dq, a.dk, a.dv = _tensor(dq), _tensor(dk), _tensor(dv)
    a.mask = _mask(mask_kind, causal_shift, kv_valid, window, frozen_keys, key_bias, _bias_shape(q, k))
    return a


def fa_bwd_workspace_bytes(q, k, *, mask_kind=FULL, key_bias=None):
    """Scratch bytes fa_bwd needs for these shapes (linear in Sq and Skv)."""
    a = _lib.fa_bwd_args()
    B, Hq, Hkv, Sq, Skv, D = _shape(q, k)
    a.dtype = _dtype_code(q)
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = B, Hq, Hkv, Sq, Skv, D
    a.mask = _mask(mask_kind, 0, None, (0, 0), 0, key_bias, _bias_shape(q, k))
    return int(_lib.lib().fa_bwd_workspace_bytes(a))


def fa_bwd(q, k, v, o, lse, dout, *, mask_kind=FULL, causal_shift=0, kv_valid=None, window=None,
           scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None, frozen_keys=0, key_bias=None):
    """Backward attention.  Returns (dQ, dK, dV) in q's dtype."""
    if dq is None:
        dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    if dk is None:
        dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    if dv is None:
        dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    a = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, mask_kind, causal_shift, kv_valid, scale, window,
                  frozen_keys, key_bias)
    need = int(_lib.lib().fa_bwd_workspace_bytes(a))
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    ws_ptr = workspace.data_ptr()
    _lib.check(_lib.lib().fa_bwd(a, ws_ptr, workspace.numel() * workspace.element_size(),
                                 _stream(q, stream)))
    return dq, dk, dv


def fa_bwd_stage(stage, q, k, v, o, lse, dout, dq, dk, dv, workspace, *, mask_kind=FULL,
                 causal_shift=0, kv_valid=None, window=None, scale=None, stream=None, frozen_keys=0,
                 key_bias=None):
    """One stage (FA_BWD_DELTA, FA_BWD_DKDV or FA_BWD_DQ) of ``fa_bwd``.

    The caller provides the outputs and the workspace; DKDV and DQ read the
    Delta (and scaled key bias) that a DELTA stage left in ``workspace``.
    """
    a = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, mask_kind, causal_shift, kv_valid, scale, window,
                  frozen_keys, key_bias)
    _lib.check(_lib.lib().fa_bwd_stage(a, int(stage), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(q, stream)))


def fa_last_error():
    return _lib.last_error()


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, mask_kind, causal_shift, kv_valid, scale, window, frozen_keys, key_bias):
        o, lse = fa_fwd(q, k, v, mask_kind=mask_kind, causal_shift=causal_shift,
                        kv_valid=kv_valid, window=window, scale=scale, key_bias=key_bias)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (mask_kind, causal_shift, kv_valid, scale, window, frozen_keys, key_bias)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        mask_kind, causal_shift, kv_valid, scale, window, frozen_keys, key_bias = ctx.cfg
        if do.stride(-1) != 1:
            do = do.contiguous()
        dq, dk, dv = fa_bwd(q, k, v, o, lse, do, mask_kind=mask_kind, causal_shift=causal_shift,
                            kv_valid=kv_valid, window=window, scale=scale, frozen_keys=frozen_keys,
                            key_bias=key_bias)
        return dq, dk, dv, None, None, None, None, None, None, None


def attention(q, k, v, mask_kind=FULL, causal_shift=0, kv_valid=None, scale=None, window=None,
              frozen_keys=0, key_bias=None):
    """Fused attention O = softmax(scale q k^T + mask) v, differentiable.

    ``scale`` defaults to 1/sqrt(D); ``window`` = (left, right) for WINDOW.
    A negative ``causal_shift`` -P with CAUSAL shows every query a P-key
    prefix; ``frozen_keys`` = P then leaves the prefix's dK, dV at zero
    without computing them.  ``key_bias`` [B, Skv] (float32) is added to the
    scaled scores; it gets no gradient.  Saves only O and LSE for the backward.
    """
    return _Attention.apply(q, k, v, mask_kind, causal_shift, kv_valid, scale, window, frozen_keys,
                            key_bias)


# ---- soft-target log-softmax loss (fa_lsm_loss_fwd / fa_lsm_loss_bwd) -------

def _loss_args(logits, target, mask):
    if logits.dim() != 2 or target.shape != logits.shape:
        raise FAError(_lib.FA_ERR_INVALID_ARG, "logits and target must be [N, V] of one shape")
    for name, t in (("logits", logits), ("target", target)):
        if t.dtype != torch.float32:
            raise FAError(_lib.FA_ERR_UNSUPPORTED, f"{name} must be float32")
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise FAError(_lib.FA_ERR_INVALID_ARG, f"{name}: the vocabulary dimension must have unit stride")
    a = _lib.fa_lsm_loss_args()
    a.N, a.V = int(logits.shape[0]), int(logits.shape[1])
    a.logits, a.logits_ss = logits.data_ptr(), logits.stride(0)
    a.target, a.target_ss = target.data_ptr(), target.stride(0)
    if mask is not None:
        if mask.dtype != torch.float32 or not mask.is_contiguous() or mask.numel() != a.N:
            raise FAError(_lib.FA_ERR_INVALID_ARG, "mask must be a contiguous float32 tensor of N elements")
        a.mask = mask.data_ptr()
    return a


def lsm_loss_fwd(logits, target, mask=None, *, stream=None):
    """Soft-target log-softmax loss (fp32).  Returns (loss [1], row_loss [N],
    m [N], d [N], tsum [N]); see fa_lsm_loss_fwd in include/fa.h."""
    N = logits.shape[0]
    a = _loss_args(logits, target, mask)
    f = lambda n: torch.empty(n, dtype=torch.float32, device=logits.device)
    loss, row, m, d, tsum = f(1), f(N), f(N), f(N), f(N)
    a.m, a.d, a.tsum, a.row_loss, a.loss = m.data_ptr(), d.data_ptr(), tsum.data_ptr(), row.data_ptr(), loss.data_ptr()
    _lib.check(_lib.lib().fa_lsm_loss_fwd(a, _stream(logits, stream)))
    return loss, row, m, d, tsum


def lsm_loss_bwd(logits, target, mask, m, d, tsum, grad_loss, *, stream=None):
    """Overwrites ``logits`` with grad_loss * dloss/dlogits and returns it."""
    a = _loss_args(logits, target, mask)
    for t in (m, d, tsum, grad_loss):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise FAError(_lib.FA_ERR_INVALID_ARG, "m, d, tsum and grad_loss must be contiguous float32")
    a.m, a.d, a.tsum, a.grad_loss = m.data_ptr(), d.data_ptr(), tsum.data_ptr(), grad_loss.data_ptr()
    _lib.check(_lib.lib().fa_lsm_loss_bwd(a, _stream(logits, stream)))
    return logits


class _LogSoftmaxLoss(torch.autograd.Function):
    """The loss as an autograd function that keeps no gradient buffer of its
    own: the backward writes the gradient over the saved logits (detached, as
    the SpecForge page's LogSoftmaxLoss does) and returns that tensor."""

    @staticmethod
    def forward(ctx, logits, target, mask):
        loss, _row, m, d, tsum = lsm_loss_fwd(logits, target, mask)
        ctx.save_for_backward(logits.detach(), target, m, d, tsum)
        ctx.mask = mask
        return loss.reshape(())

    @staticmethod
    def backward(ctx, g):
        logits, target, m, d, tsum = ctx.saved_tensors
        g = g.reshape(1).to(torch.float32).contiguous()
        return lsm_loss_bwd(logits, target, ctx.mask, m, d, tsum, g), None, None


def logsoftmax_loss(logits, target, mask=None):
    """-mean over rows of mask * sum_v target * log_softmax(logits), with the
    gradient written over ``logits``' storage in the backward (so ``logits``
    must not be needed after the backward)."""
    return _LogSoftmaxLoss.apply(logits, target, mask)
