"""ctypes view of the C ABI in include/fa.h (argument marshalling only).

Loads ``libfa.so`` from this package directory and fails loudly if it is
missing: there is no other implementation to fall back to.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_ALIGNMENT = 3
FA_ERR_ALIAS = 4
FA_ERR_HIP = 5
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED",
                3: "FA_ERR_ALIGNMENT", 4: "FA_ERR_ALIAS", 5: "FA_ERR_HIP"}

FA_BF16 = 0
FA_F32 = 1
FA_MASK_FULL = 0
FA_MASK_CAUSAL = 1
FA_MASK_TTT = 2
FA_MASK_WINDOW = 3

EXPORTED = ("fa_fwd", "fa_fwd_workspace_bytes", "fa_fwd_noalloc", "fa_bwd", "fa_bwd_stage",
            "fa_bwd_workspace_bytes", "fa_last_error", "fa_lsm_loss_fwd", "fa_lsm_loss_bwd")

# Bytes of the static device array fa_fwd_noalloc takes its workspace from
# (FA_FWD_NOALLOC_SCRATCH_BYTES in include/fa.h).
FWD_NOALLOC_SCRATCH_BYTES = 64 << 20


FA_BWD_DELTA, FA_BWD_DKDV, FA_BWD_DQ = 0, 1, 2


class fa_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_s", ctypes.c_int64)]


class fa_mask_desc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("causal_shift", ctypes.c_int32),
                ("kv_valid", ctypes.c_void_p), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32), ("frozen_keys", ctypes.c_int32),
                ("key_bias", ctypes.c_void_p), ("key_bias_stride_b", ctypes.c_int64)]


_SHAPE = [("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Hq", ctypes.c_int32),
          ("Hkv", ctypes.c_int32), ("Sq", ctypes.c_int32), ("Skv", ctypes.c_int32),
          ("D", ctypes.c_int32), ("scale", ctypes.c_float)]


class fa_fwd_args(ctypes.Structure):
    _fields_ = _SHAPE + [("q", fa_tensor), ("k", fa_tensor), ("v", fa_tensor),
                         ("o", fa_tensor), ("lse", ctypes.c_void_p),
                         ("mask", fa_mask_desc)]


class fa_bwd_args(ctypes.Structure):
    _fields_ = _SHAPE + [("q", fa_tensor), ("k", fa_tensor), ("v", fa_tensor),
                         ("o", fa_tensor), ("dout", fa_tensor), ("lse", ctypes.c_void_p),
                         ("dq", fa_tensor), ("dk", fa_tensor), ("dv", fa_tensor),
                         ("mask", fa_mask_desc)]


class fa_lsm_loss_args(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("V", ctypes.c_int32),
                ("logits", ctypes.c_void_p), ("logits_ss", ctypes.c_int64),
                ("target", ctypes.c_void_p), ("target_ss", ctypes.c_int64),
                ("mask", ctypes.c_void_p), ("m", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("tsum", ctypes.c_void_p), ("row_loss", ctypes.c_void_p), ("loss", ctypes.c_void_p),
                ("grad_loss", ctypes.c_void_p)]


class FAError(RuntimeError):
    """A non-OK status from the library, with its fa_last_error() text."""

    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded libfa.so (loaded once).  Raises if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m flash_attention_fa_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.fa_fwd.argtypes = [ctypes.POINTER(fa_fwd_args), ctypes.c_void_p,
                             ctypes.c_size_t, ctypes.c_void_p]
        L.fa_fwd.restype = ctypes.c_int
        L.fa_fwd_noalloc.argtypes = [ctypes.POINTER(fa_fwd_args), ctypes.c_void_p]
        L.fa_fwd_noalloc.restype = ctypes.c_int
        L.fa_fwd_workspace_bytes.argtypes = [ctypes.POINTER(fa_fwd_args)]
        L.fa_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.fa_bwd.argtypes = [ctypes.POINTER(fa_bwd_args), ctypes.c_void_p,
                             ctypes.c_size_t, ctypes.c_void_p]
        L.fa_bwd.restype = ctypes.c_int
        L.fa_bwd_stage.argtypes = [ctypes.POINTER(fa_bwd_args), ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
        L.fa_bwd_stage.restype = ctypes.c_int
        L.fa_bwd_workspace_bytes.argtypes = [ctypes.POINTER(fa_bwd_args)]
        L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        for name in ("fa_lsm_loss_fwd", "fa_lsm_loss_bwd"):
            getattr(L, name).argtypes = [ctypes.POINTER(fa_lsm_loss_args), ctypes.c_void_p]
            getattr(L, name).restype = ctypes.c_int
        L.fa_last_error.argtypes = []
        L.fa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error():
    return lib().fa_last_error().decode()


def check(status):
    if status != FA_OK:
        raise FAError(status, last_error())
