"""fp64 CPU oracle for the sparse-routed gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library; the arithmetic lives in the C sources beside this file
(each function there cites the slide it follows) and this module only
marshals numpy arrays.

Functions
---------
sdm_address     product-key addressing (Sparse Delta Memory slides,
                "Product keys select addresses without scoring every slot")
sdm_recurrence  sparse decay / delta update / read given the addressing
                (Sparse Delta Memory slides, Eqs. (3)-(5) and the
                shared-prediction figure form)
sdm_forward     addressing for writes and reads, then the recurrence
sdm_recurrence_backward  gradient of the recurrence by undoing writes (same
                slides, backup "Backup: undoing writes avoids repeated
                full-table snapshots")
sdm_address_backward     gradient of the addressing softmax w.r.t. the halves
sdm_backward    both, for the whole SDM forward
norm_gate       RMS-Norm and output gate after the read (same slides, the
                note after Eqs. (3)-(5))
gdn             sequential Gated DeltaNet / KDA (Linear Attention
                Architectures slides, Eqs. 14-20)
gdn2            sequential GDN2: key-side erase b, value-side write w
                (same slides, Eqs. 21-24)
sse             Sparse State Expansion per-token definition, or its masking
                execution (Sparse State Expansion slides, Eqs. (9)-(14))
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


class _Nullable:
    """ctypes argtype accepting None (NULL) or a C-contiguous array of one dtype."""

    def __init__(self, dtype):
        self.dtype = np.dtype(dtype)

    def from_param(self, obj):
        if obj is None:
            return None
        if not isinstance(obj, np.ndarray) or obj.dtype != self.dtype or not obj.flags.c_contiguous:
            raise TypeError(f"expected C-contiguous {self.dtype} array")
        return obj.ctypes.data_as(ctypes.c_void_p)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # noqa: F401  (build only when nothing is built)
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_sdm_address.restype = ctypes.c_int
    lib.orc_sdm_address.argtypes = [ctypes.c_int, ctypes.c_int, _f32p, _f32p, ctypes.c_int,
                                    ctypes.c_int, _i32p, _f64p]
    lib.orc_sdm_recurrence.restype = ctypes.c_int
    lib.orc_sdm_recurrence.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_longlong,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       _i32p, _f64p, _i32p, _f64p, _f32p, _f32p, _f32p, _f64p, _f64p]
    lib.orc_sdm_recurrence_backward.restype = ctypes.c_int
    lib.orc_sdm_recurrence_backward.argtypes = (
        [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
         ctypes.c_int, ctypes.c_int, _i32p, _f64p, _i32p, _f64p, _f32p, _f32p, _f32p]
        + [_f64p] * 8)
    lib.orc_sdm_address_backward.restype = ctypes.c_int
    lib.orc_sdm_address_backward.argtypes = [ctypes.c_int] * 3 + [_i32p, _f64p, _f64p, _f64p,
                                                                  _f64p]
    lib.orc_norm_gate.restype = ctypes.c_int
    lib.orc_norm_gate.argtypes = [ctypes.c_int, ctypes.c_int, _f32p, _Nullable(np.float32), _f32p,
                                  ctypes.c_double, ctypes.c_int, _f64p]
    lib.orc_gdn.restype = ctypes.c_int
    lib.orc_gdn.argtypes = [ctypes.c_int] * 6 + [_f32p, _f32p, _f32p, _f32p, _f32p,
                                                 _Nullable(np.float64), _f64p, _f64p]
    lib.orc_gdn2.restype = ctypes.c_int
    lib.orc_gdn2.argtypes = [ctypes.c_int] * 5 + [_f32p] * 6 + [_Nullable(np.float64), _f64p, _f64p]
    lib.orc_sse.restype = ctypes.c_int
    lib.orc_sse.argtypes = [ctypes.c_int] * 7 + [_f32p, _f32p, _f32p, _f32p, _f32p,
                                                 _Nullable(np.float32), _Nullable(np.float32),
                                                 _f64p, _f64p, _Nullable(np.int32),
                                                 _Nullable(np.float64), ctypes.c_int]
    _lib = lib
    return lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def sdm_address(s1, s2, k, budget):
    """Product-key addressing.  s1, s2: [..., sqrtN] fp32 half scores.

    Returns (idx int32 [..., budget] in rank order, wt float64 [..., budget]).
    """
    s1, s2 = _f32(s1), _f32(s2)
    assert s1.shape == s2.shape
    lead, sqrt_n = s1.shape[:-1], s1.shape[-1]
    p = int(np.prod(lead)) if lead else 1
    idx = np.empty(lead + (budget,), np.int32)
    wt = np.empty(lead + (budget,), np.float64)
    rc = _load().orc_sdm_address(p, sqrt_n, s1, s2, int(k), int(budget), idx, wt)
    if rc != 0:
        raise ValueError("orc_sdm_address: invalid arguments")
    return idx, wt


def sdm_recurrence(idx_w, wt_w, idx_r, wt_r, v, alpha, beta, M0, residual_mode=0):
    """SDM recurrence given the addressing.

    idx_w, wt_w: [B,T,H,W]; idx_r, wt_r: [B,T,H,R]; v: [B,T,H,dv];
    alpha, beta: [B,T,H]; M0: [B,H,N,dv] (not modified).
    Returns (M float64 [B,H,N,dv], y float64 [B,T,H,dv]).
    """
    idx_w = np.ascontiguousarray(idx_w, np.int32)
    idx_r = np.ascontiguousarray(idx_r, np.int32)
    wt_w = np.ascontiguousarray(wt_w, np.float64)
    wt_r = np.ascontiguousarray(wt_r, np.float64)
    v, alpha, beta = _f32(v), _f32(alpha), _f32(beta)
    B, T, H, W = idx_w.shape
    R = idx_r.shape[-1]
    dv = v.shape[-1]
    M = np.array(M0, dtype=np.float64, order="C", copy=True)
    N = M.shape[2]
    y = np.zeros((B, T, H, dv), np.float64)
    rc = _load().orc_sdm_recurrence(B, T, H, N, dv, W, R, int(residual_mode), idx_w, wt_w, idx_r,
                                    wt_r, v, alpha, beta, M, y)
    if rc != 0:
        raise ValueError("orc_sdm_recurrence: invalid arguments")
    return M, y


def sdm_forward(sw1, sw2, sr1, sr2, v, alpha, beta, M0, k_w, k_r, W, R, residual_mode=0):
    """Addressing for writes (sw1, sw2) and reads (sr1, sr2), then the recurrence.

    Score halves: [B,T,H,sqrtN].  Returns dict with M, y, idx_w, wt_w, idx_r, wt_r.
    """
    idx_w, wt_w = sdm_address(sw1, sw2, k_w, W)
    idx_r, wt_r = sdm_address(sr1, sr2, k_r, R)
    M, y = sdm_recurrence(idx_w, wt_w, idx_r, wt_r, v, alpha, beta, M0, residual_mode)
    return dict(M=M, y=y, idx_w=idx_w, wt_w=wt_w, idx_r=idx_r, wt_r=wt_r)


def sdm_recurrence_backward(idx_w, wt_w, idx_r, wt_r, v, alpha, beta, M0, dy, dM=None,
                            residual_mode=0):
    """Gradient of sdm_recurrence by undoing writes.

    dy: [B,T,H,dv] gradient of y; dM: [B,H,N,dv] gradient of the final table
    (None = zeros).  Returns dict with dv [B,T,H,dv], dalpha, dbeta [B,T,H],
    dwt_w [B,T,H,W], dwt_r [B,T,H,R] and dM0 [B,H,N,dv] (gradient of M0), all
    float64.
    """
    idx_w = np.ascontiguousarray(idx_w, np.int32)
    idx_r = np.ascontiguousarray(idx_r, np.int32)
    wt_w = np.ascontiguousarray(wt_w, np.float64)
    wt_r = np.ascontiguousarray(wt_r, np.float64)
    v, alpha, beta = _f32(v), _f32(alpha), _f32(beta)
    B, T, H, W = idx_w.shape
    R = idx_r.shape[-1]
    dvw = v.shape[-1]
    M0 = np.ascontiguousarray(M0, np.float64)
    N = M0.shape[2]
    dy = np.ascontiguousarray(dy, np.float64)
    G = np.zeros(M0.shape, np.float64) if dM is None else np.array(dM, np.float64, order="C")
    out = dict(dv=np.zeros((B, T, H, dvw)), dalpha=np.zeros((B, T, H)),
               dbeta=np.zeros((B, T, H)), dwt_w=np.zeros((B, T, H, W)),
               dwt_r=np.zeros((B, T, H, R)))
    rc = _load().orc_sdm_recurrence_backward(B, T, H, N, dvw, W, R, int(residual_mode), idx_w,
                                             wt_w, idx_r, wt_r, v, alpha, beta, M0, dy, G,
                                             out["dv"], out["dalpha"], out["dbeta"],
                                             out["dwt_w"], out["dwt_r"])
    if rc != 0:
        raise ValueError("orc_sdm_recurrence_backward: invalid arguments")
    out["dM0"] = G
    return out


def sdm_address_backward(idx, wt, dwt, sqrt_n):
    """Gradient of the addressing softmax, selection held fixed.

    idx, wt, dwt: [..., budget].  Returns (ds1, ds2) float64 [..., sqrtN].
    """
    idx = np.ascontiguousarray(idx, np.int32)
    wt = np.ascontiguousarray(wt, np.float64)
    dwt = np.ascontiguousarray(dwt, np.float64)
    lead, budget = idx.shape[:-1], idx.shape[-1]
    p = int(np.prod(lead)) if lead else 1
    ds1 = np.zeros(lead + (sqrt_n,))
    ds2 = np.zeros(lead + (sqrt_n,))
    rc = _load().orc_sdm_address_backward(p, int(sqrt_n), budget, idx, wt, dwt, ds1, ds2)
    if rc != 0:
        raise ValueError("orc_sdm_address_backward: invalid arguments")
    return ds1, ds2


def sdm_backward(sw1, sw2, sr1, sr2, v, alpha, beta, M0, k_w, k_r, W, R, dy, dM=None,
                 residual_mode=0):
    """Gradient of sdm_forward w.r.t. every input: the recurrence by undoing
    writes, then the addressing softmax (selection fixed).  Returns the dict of
    sdm_recurrence_backward plus dsw1, dsw2, dsr1, dsr2 [B,T,H,sqrtN]."""
    sqrt_n = np.shape(sw1)[-1]
    idx_w, wt_w = sdm_address(sw1, sw2, k_w, W)
    idx_r, wt_r = sdm_address(sr1, sr2, k_r, R)
    g = sdm_recurrence_backward(idx_w, wt_w, idx_r, wt_r, v, alpha, beta, M0, dy, dM,
                                residual_mode)
    g["dsw1"], g["dsw2"] = sdm_address_backward(idx_w, wt_w, g["dwt_w"], sqrt_n)
    g["dsr1"], g["dsr2"] = sdm_address_backward(idx_r, wt_r, g["dwt_r"], sqrt_n)
    return g


ACTS = {"none": 0, "silu": 1, "sigmoid": 2}


def norm_gate(y, g, gamma, eps=1e-6, act="silu"):
    """o = y / sqrt(mean(y^2) + eps) * gamma * act(g) over the last axis.

    y, g: [..., d] (g may be None when act == "none"); gamma: [d].  float64 out."""
    y = _f32(y)
    d = y.shape[-1]
    p = int(np.prod(y.shape[:-1])) if y.ndim > 1 else 1
    g = None if g is None else _f32(g)
    if g is None and act != "none":
        raise ValueError("a gate is needed unless act == 'none'")
    o = np.zeros(y.shape, np.float64)
    rc = _load().orc_norm_gate(p, d, y, g, _f32(gamma), float(eps), ACTS[act], o)
    if rc != 0:
        raise ValueError("orc_norm_gate: invalid arguments")
    return o


def gdn(q, k, v, alpha, beta, S0=None, kda=False):
    """Sequential GDN (alpha [B,T,H]) or KDA (alpha [B,T,H,dk]).

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H]; S0: [B,H,dk,dv] or None.
    Returns (S float64 [B,H,dk,dv], o float64 [B,T,H,dv]).
    """
    q, k, v, alpha, beta = _f32(q), _f32(k), _f32(v), _f32(alpha), _f32(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv), np.float64)
    o = np.zeros((B, T, H, dv), np.float64)
    s0 = None if S0 is None else np.ascontiguousarray(S0, np.float64)
    rc = _load().orc_gdn(B, T, H, dk, dv, 1 if kda else 0, q, k, v, alpha, beta, s0, S, o)
    if rc != 0:
        raise ValueError("orc_gdn: invalid arguments")
    return S, o


def gdn2(q, k, v, alpha, b, w, S0=None):
    """Sequential GDN2: per-channel decay alpha and erase vector b [B,T,H,dk], write
    vector w [B,T,H,dv] (slide "GDN2 separates key-side erase and value-side write").

    Returns (S float64 [B,H,dk,dv], o float64 [B,T,H,dv]).
    """
    q, k, v, alpha, b, w = _f32(q), _f32(k), _f32(v), _f32(alpha), _f32(b), _f32(w)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv), np.float64)
    o = np.zeros((B, T, H, dv), np.float64)
    s0 = None if S0 is None else np.ascontiguousarray(S0, np.float64)
    rc = _load().orc_gdn2(B, T, H, dk, dv, q, k, v, alpha, b, w, s0, S, o)
    if rc != 0:
        raise ValueError("orc_gdn2: invalid arguments")
    return S, o


def sse(logits, q, k, v, lam, topk, q_sh=None, k_sh=None, S0=None, masking=False):
    """Sparse State Expansion forward.

    logits: [B,T,H,N]; q, k, lam: [B,T,H,c]; v: [B,T,H,d]; S0: [B,H,N+1,c,d] or None.
    Returns dict with S float64 [B,H,N+1,c,d], o float64 [B,T,H,d], sel int32 and
    e_sel float64 [B,T,H,topk].
    """
    logits, q, k, v, lam = _f32(logits), _f32(q), _f32(k), _f32(v), _f32(lam)
    B, T, H, N = logits.shape
    c, d = q.shape[-1], v.shape[-1]
    if S0 is None:
        S = np.zeros((B, H, N + 1, c, d), np.float64)
    else:
        S = np.array(S0, dtype=np.float64, order="C", copy=True)
    o = np.zeros((B, T, H, d), np.float64)
    sel = np.zeros((B, T, H, topk), np.int32)
    e_sel = np.zeros((B, T, H, topk), np.float64)
    qs = None if q_sh is None else _f32(q_sh)
    ks = None if k_sh is None else _f32(k_sh)
    rc = _load().orc_sse(B, T, H, N, int(topk), c, d, logits, q, k, v, lam, qs, ks, S, o, sel,
                         e_sel, 1 if masking else 0)
    if rc != 0:
        raise ValueError("orc_sse: invalid arguments")
    return dict(S=S, o=o, sel=sel, e_sel=e_sel)
