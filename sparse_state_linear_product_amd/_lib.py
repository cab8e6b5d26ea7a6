"""ctypes loader for libsslp.so and the C shape structs of include/sslp.h.

The library is loaded from this package directory only.  There is no
fallback: if libsslp.so has not been built, loading raises.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsslp.so")

SSLP_OK = 0
SSLP_ERR_INVALID_ARG = -1
SSLP_ERR_UNSUPPORTED = -2
SSLP_ERR_WORKSPACE = -3
SSLP_ERR_HIP = -4

SSLP_FP32 = 0
SSLP_BF16 = 1
RESIDUAL_SHARED = 0
RESIDUAL_PER_SLOT = 1
DECAY_SCALAR = 0
DECAY_CHANNEL = 1


class SdmShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "T", "H", "sqrtN", "d_v", "k_w", "k_r", "W", "R")]


class GdnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "T", "H", "d_k", "d_v", "chunk")]


class SseShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "T", "H", "N", "topk", "c", "d", "chunk")]


# exported symbols and their C signatures (argument ctypes, return ctypes)
_vp, _sz, _i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
SIGNATURES = {
    "sdm_workspace_size": ([ctypes.POINTER(SdmShape)], _sz),
    "sdm_decode_workspace_size": ([ctypes.POINTER(SdmShape)], _sz),
    "sdm_forward": ([ctypes.POINTER(SdmShape), _i, _i] + [_vp] * 14 + [_sz, _vp], _i),
    "sdm_decode_step": ([ctypes.POINTER(SdmShape), _i, _i] + [_vp] * 14 + [_sz, _vp], _i),
    "sdm_noalloc_scratch_bytes": ([], _sz),
    "sdm_forward_noalloc": ([ctypes.POINTER(SdmShape), _i, _i] + [_vp] * 14, _i),
    "sdm_address": ([ctypes.POINTER(SdmShape), _i, _vp, _vp, _i, _i, _vp, _vp, _vp], _i),
    "sdm_sparse_update": ([ctypes.POINTER(SdmShape), _i, _i] + [_vp] * 10 + [_sz, _vp], _i),
    "sdm_norm_gate": ([ctypes.c_longlong, _i, _i, _vp, _vp, _vp, ctypes.c_float, _i, _vp, _vp],
                      _i),
    "sdm_forward_train": ([ctypes.POINTER(SdmShape), _i, _i] + [_vp] * 15 + [_sz, _vp], _i),
    "sdm_sparse_update_train": ([ctypes.POINTER(SdmShape), _i, _i] + [_vp] * 11 + [_sz, _vp],
                                _i),
    "sdm_train_workspace_size": ([ctypes.POINTER(SdmShape)], _sz),
    "sdm_backward_workspace_size": ([ctypes.POINTER(SdmShape)], _sz),
    "sdm_backward": ([ctypes.POINTER(SdmShape), _i, _i] + [_vp] * 21 + [_sz, _vp], _i),
    "gdn_workspace_size": ([ctypes.POINTER(GdnShape)], _sz),
    "gdn_chunk_forward": ([ctypes.POINTER(GdnShape), _i, _i] + [_vp] * 9 + [_sz, _vp], _i),
    "gdn2_chunk_forward": ([ctypes.POINTER(GdnShape), _i] + [_vp] * 10 + [_sz, _vp], _i),
    "sse_workspace_size": ([ctypes.POINTER(SseShape)], _sz),
    "sse_forward": ([ctypes.POINTER(SseShape), _i] + [_vp] * 12 + [_sz, _vp], _i),
    "sse_forward_masking": ([ctypes.POINTER(SseShape), _i] + [_vp] * 12 + [_sz, _vp], _i),
    "sse_decode_step": ([ctypes.POINTER(SseShape), _i] + [_vp] * 11 + [_vp], _i),
    "sslp_last_error": ([], ctypes.c_char_p),
    "sslp_device_error": ([_vp], _i),
    "sslp_version": ([], _i),
}

_lib = None


def lib():
    """The loaded libsslp.so (raises OSError/FileNotFoundError when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`"
                " or `python sparse_state_linear_product_amd/build.py`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (argtypes, restype) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = handle
    return _lib


class SslpError(RuntimeError):
    def __init__(self, fn, code):
        msg = lib().sslp_last_error().decode(errors="replace")
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def check(fn, code):
    if code != SSLP_OK:
        raise SslpError(fn, code)
