"""Sparse-routed gated delta-rule recurrence on AMD MI355X (gfx950).

Thin Python binding over libsslp.so (include/sslp.h).  Each function takes
torch tensors that already live on the GPU, checks their dtype, shape and
contiguity, and passes raw device pointers plus the current HIP stream to the
C function of the same name; every step of the computation runs in the HIP
kernels.  PyTorch provides device memory and streams only.  Workspaces are
allocated with torch when the caller does not pass one, on the stream the
call is enqueued on.

Functions (see include/sslp.h for the exact semantics):
  sdm_forward, sdm_decode_step, sdm_address, sdm_sparse_update   Sparse Delta Memory
  sdm_forward_noalloc                                            the same, with the library's fixed scratch
  sdm_norm_gate                                                  RMS-Norm + output gate after the read
  sdm_forward_train, sdm_sparse_update_train, sdm_backward       SDM training (undo writes)
  gdn_chunk_forward, gdn2_chunk_forward                          Gated DeltaNet / KDA / GDN2
  sse_forward (masking=True: sse_forward_masking), sse_decode_step  Sparse State Expansion
"""
import contextlib
import ctypes

import torch

from . import _lib
from ._lib import (DECAY_CHANNEL, DECAY_SCALAR, RESIDUAL_PER_SLOT, RESIDUAL_SHARED, GdnShape,
                   SdmShape, SseShape, SslpError, check, lib)

__all__ = ["sdm_forward", "sdm_forward_noalloc", "sdm_noalloc_scratch_bytes", "sdm_decode_step", "sdm_address", "sdm_sparse_update",
           "sdm_forward_train", "sdm_sparse_update_train", "sdm_backward",
           "sdm_train_workspace_bytes", "sdm_backward_workspace_bytes", "sdm_norm_gate",
           "gdn_chunk_forward", "gdn2_chunk_forward", "sse_forward", "sse_decode_step",
           "SslpError", "RESIDUAL_SHARED", "RESIDUAL_PER_SLOT", "DECAY_SCALAR", "DECAY_CHANNEL",
           "version", "device_error"]


def version():
    return lib().sslp_version()


def device_error(stream=None):
    """True if an SDM kernel met a caller-supplied slot index outside [0, N) since
    the last query on this device (that call's results are undefined; no memory
    outside its tensors was touched).  Synchronises the stream; clears the flag."""
    rc = lib().sslp_device_error(_stream(stream))
    if rc < 0:
        check("sslp_device_error", rc)
    return rc == 1


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return _lib.SSLP_FP32
    if t.dtype == torch.bfloat16:
        return _lib.SSLP_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream):
    """Context in which the binding's own allocations and fills (workspaces,
    outputs, zero-filled gradients) are made: the caller's stream when one is
    given, so that the caching allocator orders their reuse and the fills
    after the kernels enqueued there."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _workspace(nbytes, workspace, device):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace must hold {nbytes} bytes")
        return workspace, workspace.numel() * workspace.element_size()
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


# ---------------------------------------------------------------------------
# Sparse Delta Memory
# ---------------------------------------------------------------------------
def sdm_shape(B, T, H, sqrtN, d_v, k_w, k_r, W, R):
    return SdmShape(B, T, H, sqrtN, d_v, k_w, k_r, W, R)


def sdm_workspace_size(shape):
    return lib().sdm_workspace_size(ctypes.byref(shape))


def sdm_forward(sw1, sw2, sr1, sr2, v, alpha, beta, M, k_w, k_r, W, R, y=None,
                residual_mode=RESIDUAL_SHARED, idx_w=None, wt_w=None, idx_r=None, wt_r=None,
                workspace=None, stream=None):
    """Addressing + recurrence over T tokens; M [B,H,N,d_v] fp32 is updated in place.

    sw1, sw2, sr1, sr2: [B,T,H,sqrtN]; v: [B,T,H,d_v] (same dtype); alpha, beta: [B,T,H]
    fp32.  Returns y [B,T,H,d_v] (allocated if not given)."""
    with _on_stream(stream):
        B, T, H, sqrt_n = sw1.shape
        d_v = v.shape[-1]
        dt = sw1.dtype
        for name, t in (("sw2", sw2), ("sr1", sr1), ("sr2", sr2)):
            _need(t, dt, (B, T, H, sqrt_n), name)
        _need(v, dt, (B, T, H, d_v), "v")
        _need(alpha, torch.float32, (B, T, H), "alpha")
        _need(beta, torch.float32, (B, T, H), "beta")
        _need(M, torch.float32, (B, H, sqrt_n * sqrt_n, d_v), "M")
        if y is None:
            y = torch.empty((B, T, H, d_v), dtype=dt, device=v.device)
        _need(y, dt, (B, T, H, d_v), "y")
        shape = sdm_shape(B, T, H, sqrt_n, d_v, k_w, k_r, W, R)
        ws, nbytes = _workspace(lib().sdm_workspace_size(ctypes.byref(shape)), workspace, v.device)
        rc = lib().sdm_forward(ctypes.byref(shape), _dtype_code(sw1), int(residual_mode), _ptr(sw1),
                               _ptr(sw2), _ptr(sr1), _ptr(sr2), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(M), _ptr(y), _ptr(idx_w), _ptr(wt_w), _ptr(idx_r), _ptr(wt_r),
                               _ptr(ws), nbytes, _stream(stream))
        check("sdm_forward", rc)
        return y


def sdm_noalloc_scratch_bytes():
    """Fixed per-GPU scratch of sdm_forward_noalloc, in bytes."""
    return lib().sdm_noalloc_scratch_bytes()


def sdm_forward_noalloc(sw1, sw2, sr1, sr2, v, alpha, beta, M, y, k_w, k_r, W, R,
                        residual_mode=RESIDUAL_SHARED, idx_w=None, wt_w=None, idx_r=None,
                        wt_r=None, stream=None):
    """sdm_forward with no workspace and no allocation anywhere in the call: y
    [B,T,H,d_v] must be given; the scratch is the library's fixed per-GPU array
    (calls that overlap on one GPU race).  Returns y."""
    with _on_stream(stream):
        B, T, H, sqrt_n = sw1.shape
        d_v = v.shape[-1]
        dt = sw1.dtype
        for name, t in (("sw2", sw2), ("sr1", sr1), ("sr2", sr2)):
            _need(t, dt, (B, T, H, sqrt_n), name)
        _need(v, dt, (B, T, H, d_v), "v")
        _need(alpha, torch.float32, (B, T, H), "alpha")
        _need(beta, torch.float32, (B, T, H), "beta")
        _need(M, torch.float32, (B, H, sqrt_n * sqrt_n, d_v), "M")
        _need(y, dt, (B, T, H, d_v), "y")
        for name, t, n in (("idx_w", idx_w, W), ("idx_r", idx_r, R)):
            if t is not None:
                _need(t, torch.int32, (B, T, H, n), name)
        for name, t, n in (("wt_w", wt_w, W), ("wt_r", wt_r, R)):
            if t is not None:
                _need(t, torch.float32, (B, T, H, n), name)
        shape = sdm_shape(B, T, H, sqrt_n, d_v, k_w, k_r, W, R)
        rc = lib().sdm_forward_noalloc(ctypes.byref(shape), _dtype_code(sw1), int(residual_mode),
                                       _ptr(sw1), _ptr(sw2), _ptr(sr1), _ptr(sr2), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(M), _ptr(y), _ptr(idx_w),
                                       _ptr(wt_w), _ptr(idx_r), _ptr(wt_r), _stream(stream))
        check("sdm_forward_noalloc", rc)
        return y


def sdm_decode_step(sw1, sw2, sr1, sr2, v, alpha, beta, M, k_w, k_r, W, R, y=None,
                    residual_mode=RESIDUAL_SHARED, idx_w=None, wt_w=None, idx_r=None, wt_r=None,
                    workspace=None, stream=None):
    """One token for each of B sequences.  sw*, sr*: [B,H,sqrtN]; v: [B,H,d_v];
    alpha, beta: [B,H]; M: [B,H,N,d_v] fp32 in place.  Returns y [B,H,d_v]."""
    with _on_stream(stream):
        B, H, sqrt_n = sw1.shape
        d_v = v.shape[-1]
        dt = sw1.dtype
        for name, t in (("sw2", sw2), ("sr1", sr1), ("sr2", sr2)):
            _need(t, dt, (B, H, sqrt_n), name)
        _need(v, dt, (B, H, d_v), "v")
        _need(alpha, torch.float32, (B, H), "alpha")
        _need(beta, torch.float32, (B, H), "beta")
        _need(M, torch.float32, (B, H, sqrt_n * sqrt_n, d_v), "M")
        if y is None:
            y = torch.empty((B, H, d_v), dtype=dt, device=v.device)
        _need(y, dt, (B, H, d_v), "y")
        shape = sdm_shape(B, 1, H, sqrt_n, d_v, k_w, k_r, W, R)
        ws, nbytes = _workspace(lib().sdm_decode_workspace_size(ctypes.byref(shape)), workspace,
                               v.device)
        rc = lib().sdm_decode_step(ctypes.byref(shape), _dtype_code(sw1), int(residual_mode),
                                   _ptr(sw1), _ptr(sw2), _ptr(sr1), _ptr(sr2), _ptr(v), _ptr(alpha),
                                   _ptr(beta), _ptr(M), _ptr(y), _ptr(idx_w), _ptr(wt_w), _ptr(idx_r),
                                   _ptr(wt_r), _ptr(ws), nbytes, _stream(stream))
        check("sdm_decode_step", rc)
        return y


def sdm_address(s1, s2, k, budget, idx=None, wt=None, stream=None):
    """Product-key addressing alone.  s1, s2: [B,T,H,sqrtN].  Returns (idx, wt)."""
    with _on_stream(stream):
        B, T, H, sqrt_n = s1.shape
        _need(s2, s1.dtype, s1.shape, "s2")
        if idx is None:
            idx = torch.empty((B, T, H, budget), dtype=torch.int32, device=s1.device)
        if wt is None:
            wt = torch.empty((B, T, H, budget), dtype=torch.float32, device=s1.device)
        _need(idx, torch.int32, (B, T, H, budget), "idx")
        _need(wt, torch.float32, (B, T, H, budget), "wt")
        shape = sdm_shape(B, T, H, sqrt_n, 1, 1, 1, 1, 1)
        rc = lib().sdm_address(ctypes.byref(shape), _dtype_code(s1), _ptr(s1), _ptr(s2), int(k),
                               int(budget), _ptr(idx), _ptr(wt), _stream(stream))
        check("sdm_address", rc)
        return idx, wt


def sdm_sparse_update(idx_w, wt_w, idx_r, wt_r, v, alpha, beta, M, y=None,
                      residual_mode=RESIDUAL_SHARED, workspace=None, stream=None):
    """The recurrence alone with caller-supplied addressing (raw weights)."""
    with _on_stream(stream):
        B, T, H, W = idx_w.shape
        R = idx_r.shape[-1]
        d_v = v.shape[-1]
        N = M.shape[2]
        sqrt_n = int(round(N ** 0.5))
        if sqrt_n * sqrt_n != N:
            raise ValueError("M.shape[2] must be a perfect square")
        _need(idx_w, torch.int32, (B, T, H, W), "idx_w")
        _need(wt_w, torch.float32, (B, T, H, W), "wt_w")
        _need(idx_r, torch.int32, (B, T, H, R), "idx_r")
        _need(wt_r, torch.float32, (B, T, H, R), "wt_r")
        _need(alpha, torch.float32, (B, T, H), "alpha")
        _need(beta, torch.float32, (B, T, H), "beta")
        _need(M, torch.float32, (B, H, N, d_v), "M")
        if y is None:
            y = torch.empty((B, T, H, d_v), dtype=v.dtype, device=v.device)
        _need(y, v.dtype, (B, T, H, d_v), "y")
        shape = sdm_shape(B, T, H, sqrt_n, d_v, 1, 1, W, R)
        ws, nbytes = _workspace(lib().sdm_workspace_size(ctypes.byref(shape)), workspace, v.device)
        rc = lib().sdm_sparse_update(ctypes.byref(shape), _dtype_code(v), int(residual_mode),
                                     _ptr(idx_w), _ptr(wt_w), _ptr(idx_r), _ptr(wt_r), _ptr(v),
                                     _ptr(alpha), _ptr(beta), _ptr(M), _ptr(y), _ptr(ws), nbytes,
                                     _stream(stream))
        check("sdm_sparse_update", rc)
        return y


GATE_ACTS = {"none": 0, "silu": 1, "sigmoid": 2}


def sdm_norm_gate(y, gamma, gate=None, eps=1e-6, act="silu", o=None, stream=None):
    """RMS-Norm over the last axis of y, times gamma [d] fp32 and act(gate).

    y, gate: [..., d] (same dtype, contiguous); returns o (y itself when o is y)."""
    with _on_stream(stream):
        d = y.shape[-1]
        rows = y.numel() // d if d else 0
        _need(gamma, torch.float32, (d,), "gamma")
        if gate is not None:
            _need(gate, y.dtype, tuple(y.shape), "gate")
        if o is None:
            o = torch.empty_like(y)
        _need(o, y.dtype, tuple(y.shape), "o")
        _need(y, y.dtype, tuple(y.shape), "y")
        rc = lib().sdm_norm_gate(rows, d, _dtype_code(y), _ptr(y), _ptr(gate), _ptr(gamma),
                                 float(eps), GATE_ACTS[act], _ptr(o), _stream(stream))
        check("sdm_norm_gate", rc)
        return o


def sdm_train_workspace_bytes(B, T, H, sqrtN, d_v, W, R):
    """Workspace bytes of sdm_forward_train / sdm_sparse_update_train (chunk plans)."""
    return lib().sdm_train_workspace_size(ctypes.byref(sdm_shape(B, T, H, sqrtN, d_v, 1, 1, W, R)))


def sdm_backward_workspace_bytes(B, T, H, sqrtN, d_v, W, R):
    return lib().sdm_backward_workspace_size(ctypes.byref(sdm_shape(B, T, H, sqrtN, d_v, 1, 1,
                                                                     W, R)))


def sdm_forward_train(sw1, sw2, sr1, sr2, v, alpha, beta, M, k_w, k_r, W, R, y=None,
                      residual_mode=RESIDUAL_SHARED, out=None, workspace=None, stream=None):
    """sdm_forward that keeps what sdm_backward needs.  M is updated in place.

    Returns (y, dict(idx_w, wt_w, idx_r, wt_r, saved)); saved [B,T,H,W,d_v] fp32
    holds each token's write rows as they were before the token.  `out` may pass
    such a dict of preallocated tensors to fill."""
    with _on_stream(stream):
        B, T, H, sqrt_n = sw1.shape
        d_v = v.shape[-1]
        dt = sw1.dtype
        for name, t in (("sw2", sw2), ("sr1", sr1), ("sr2", sr2)):
            _need(t, dt, (B, T, H, sqrt_n), name)
        _need(v, dt, (B, T, H, d_v), "v")
        _need(alpha, torch.float32, (B, T, H), "alpha")
        _need(beta, torch.float32, (B, T, H), "beta")
        _need(M, torch.float32, (B, H, sqrt_n * sqrt_n, d_v), "M")
        if y is None:
            y = torch.empty((B, T, H, d_v), dtype=dt, device=v.device)
        _need(y, dt, (B, T, H, d_v), "y")
        dev = v.device
        if out is None:
            out = dict(idx_w=torch.empty((B, T, H, W), dtype=torch.int32, device=dev),
                       wt_w=torch.empty((B, T, H, W), dtype=torch.float32, device=dev),
                       idx_r=torch.empty((B, T, H, R), dtype=torch.int32, device=dev),
                       wt_r=torch.empty((B, T, H, R), dtype=torch.float32, device=dev),
                       saved=torch.empty((B, T, H, W, d_v), dtype=torch.float32, device=dev))
        ctx = out
        _need(ctx["idx_w"], torch.int32, (B, T, H, W), "idx_w")
        _need(ctx["wt_w"], torch.float32, (B, T, H, W), "wt_w")
        _need(ctx["idx_r"], torch.int32, (B, T, H, R), "idx_r")
        _need(ctx["wt_r"], torch.float32, (B, T, H, R), "wt_r")
        _need(ctx["saved"], torch.float32, (B, T, H, W, d_v), "saved")
        shape = sdm_shape(B, T, H, sqrt_n, d_v, k_w, k_r, W, R)
        ws, nbytes = _workspace(lib().sdm_train_workspace_size(ctypes.byref(shape)), workspace,
                                v.device)
        rc = lib().sdm_forward_train(ctypes.byref(shape), _dtype_code(sw1), int(residual_mode),
                                     _ptr(sw1), _ptr(sw2), _ptr(sr1), _ptr(sr2), _ptr(v), _ptr(alpha),
                                     _ptr(beta), _ptr(M), _ptr(y), _ptr(ctx["idx_w"]),
                                     _ptr(ctx["wt_w"]), _ptr(ctx["idx_r"]), _ptr(ctx["wt_r"]),
                                     _ptr(ctx["saved"]), _ptr(ws), nbytes, _stream(stream))
        check("sdm_forward_train", rc)
        return y, ctx


def sdm_sparse_update_train(idx_w, wt_w, idx_r, wt_r, v, alpha, beta, M, y=None, saved=None,
                            residual_mode=RESIDUAL_SHARED, workspace=None, stream=None):
    """sdm_sparse_update that also returns saved [B,T,H,W,d_v] (pre-write rows)."""
    with _on_stream(stream):
        B, T, H, W = idx_w.shape
        R = idx_r.shape[-1]
        d_v = v.shape[-1]
        N = M.shape[2]
        sqrt_n = int(round(N ** 0.5))
        if sqrt_n * sqrt_n != N:
            raise ValueError("M.shape[2] must be a perfect square")
        _need(idx_w, torch.int32, (B, T, H, W), "idx_w")
        _need(wt_w, torch.float32, (B, T, H, W), "wt_w")
        _need(idx_r, torch.int32, (B, T, H, R), "idx_r")
        _need(wt_r, torch.float32, (B, T, H, R), "wt_r")
        _need(alpha, torch.float32, (B, T, H), "alpha")
        _need(beta, torch.float32, (B, T, H), "beta")
        _need(M, torch.float32, (B, H, N, d_v), "M")
        if y is None:
            y = torch.empty((B, T, H, d_v), dtype=v.dtype, device=v.device)
        if saved is None:
            saved = torch.empty((B, T, H, W, d_v), dtype=torch.float32, device=v.device)
        _need(y, v.dtype, (B, T, H, d_v), "y")
        _need(saved, torch.float32, (B, T, H, W, d_v), "saved")
        shape = sdm_shape(B, T, H, sqrt_n, d_v, 1, 1, W, R)
        ws, nbytes = _workspace(lib().sdm_train_workspace_size(ctypes.byref(shape)), workspace,
                                v.device)
        rc = lib().sdm_sparse_update_train(ctypes.byref(shape), _dtype_code(v), int(residual_mode),
                                           _ptr(idx_w), _ptr(wt_w), _ptr(idx_r), _ptr(wt_r), _ptr(v),
                                           _ptr(alpha), _ptr(beta), _ptr(M), _ptr(y), _ptr(saved),
                                           _ptr(ws), nbytes, _stream(stream))
        check("sdm_sparse_update_train", rc)
        return y, saved


def sdm_backward(ctx, v, alpha, beta, M, dy, dM=None, residual_mode=RESIDUAL_SHARED,
                 score_grads=True, workspace=None, stream=None):
    """Gradient of the SDM forward by undoing writes.

    ctx: the dict of sdm_forward_train (or idx_w, wt_w, idx_r, wt_r, saved of
    sdm_sparse_update_train).  M: the table after the forward, restored in place
    to the table before it.  dy [B,T,H,d_v] (dtype of v); dM [B,H,N,d_v] fp32
    gradient of the final table (zeros if None), updated in place to the
    gradient of the initial table.  Returns dict(dv, dalpha, dbeta, dwt_w, dwt_r,
    dM[, dsw1, dsw2, dsr1, dsr2]); score_grads=False skips the addressing
    backward."""
    with _on_stream(stream):
        idx_w, wt_w, idx_r, wt_r, saved = (ctx[k] for k in ("idx_w", "wt_w", "idx_r", "wt_r",
                                                             "saved"))
        B, T, H, W = idx_w.shape
        R = idx_r.shape[-1]
        d_v = v.shape[-1]
        N = M.shape[2]
        sqrt_n = int(round(N ** 0.5))
        if sqrt_n * sqrt_n != N:
            raise ValueError("M.shape[2] must be a perfect square")
        dev = v.device
        _need(idx_w, torch.int32, (B, T, H, W), "idx_w")
        _need(wt_w, torch.float32, (B, T, H, W), "wt_w")
        _need(idx_r, torch.int32, (B, T, H, R), "idx_r")
        _need(wt_r, torch.float32, (B, T, H, R), "wt_r")
        _need(alpha, torch.float32, (B, T, H), "alpha")
        _need(beta, torch.float32, (B, T, H), "beta")
        _need(M, torch.float32, (B, H, N, d_v), "M")
        _need(saved, torch.float32, (B, T, H, W, d_v), "saved")
        _need(v, v.dtype, (B, T, H, d_v), "v")
        _need(dy, v.dtype, (B, T, H, d_v), "dy")
        if dM is None:
            dM = torch.zeros((B, H, N, d_v), dtype=torch.float32, device=dev)
        _need(dM, torch.float32, (B, H, N, d_v), "dM")
        f32 = dict(dtype=torch.float32, device=dev)
        g = dict(dv=torch.empty_like(v), dalpha=torch.empty((B, T, H), **f32),
                 dbeta=torch.empty((B, T, H), **f32), dwt_w=torch.empty((B, T, H, W), **f32),
                 dwt_r=torch.empty((B, T, H, R), **f32), dM=dM)
        if score_grads:
            for k in ("dsw1", "dsw2", "dsr1", "dsr2"):
                g[k] = torch.empty((B, T, H, sqrt_n), **f32)
        shape = sdm_shape(B, T, H, sqrt_n, d_v, 1, 1, W, R)
        ws, nbytes = _workspace(lib().sdm_backward_workspace_size(ctypes.byref(shape)), workspace,
                                dev)
        rc = lib().sdm_backward(ctypes.byref(shape), _dtype_code(v), int(residual_mode), _ptr(idx_w),
                                _ptr(wt_w), _ptr(idx_r), _ptr(wt_r), _ptr(v), _ptr(alpha),
                                _ptr(beta), _ptr(M), _ptr(saved), _ptr(dy), _ptr(dM), _ptr(g["dv"]),
                                _ptr(g["dalpha"]), _ptr(g["dbeta"]), _ptr(g["dwt_w"]),
                                _ptr(g["dwt_r"]), _ptr(g.get("dsw1")), _ptr(g.get("dsw2")),
                                _ptr(g.get("dsr1")), _ptr(g.get("dsr2")), _ptr(ws), nbytes,
                                _stream(stream))
        check("sdm_backward", rc)
        return g


# ---------------------------------------------------------------------------
# Gated DeltaNet / KDA
# ---------------------------------------------------------------------------
def gdn_chunk_forward(q, k, v, alpha, beta, S0=None, S_out=None, o=None, decay_mode=None,
                      chunk=64, workspace=None, stream=None):
    """q, k: [B,T,H,d_k]; v: [B,T,H,d_v]; alpha [B,T,H] (GDN) or [B,T,H,d_k] (KDA) fp32;
    beta [B,T,H] fp32; S0 [B,H,d_k,d_v] fp32 or None.  Returns (o, S_out)."""
    with _on_stream(stream):
        B, T, H, d_k = q.shape
        d_v = v.shape[-1]
        dt = q.dtype
        _need(k, dt, (B, T, H, d_k), "k")
        _need(v, dt, (B, T, H, d_v), "v")
        if decay_mode is None:
            decay_mode = DECAY_CHANNEL if alpha.dim() == 4 else DECAY_SCALAR
        ashape = (B, T, H, d_k) if decay_mode == DECAY_CHANNEL else (B, T, H)
        _need(alpha, torch.float32, ashape, "alpha")
        _need(beta, torch.float32, (B, T, H), "beta")
        if S0 is not None:
            _need(S0, torch.float32, (B, H, d_k, d_v), "S0")
        if S_out is None:
            S_out = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=q.device)
        _need(S_out, torch.float32, (B, H, d_k, d_v), "S_out")
        if o is None:
            o = torch.empty((B, T, H, d_v), dtype=dt, device=q.device)
        _need(o, dt, (B, T, H, d_v), "o")
        shape = GdnShape(B, T, H, d_k, d_v, chunk)
        ws, nbytes = _workspace(lib().gdn_workspace_size(ctypes.byref(shape)), workspace, q.device)
        rc = lib().gdn_chunk_forward(ctypes.byref(shape), _dtype_code(q), int(decay_mode), _ptr(q),
                                     _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(S_out),
                                     _ptr(o), _ptr(ws), nbytes, _stream(stream))
        check("gdn_chunk_forward", rc)
        return o, S_out


def gdn2_chunk_forward(q, k, v, alpha, erase, write, S0=None, S_out=None, o=None, chunk=64,
                       workspace=None, stream=None):
    """GDN2: q, k [B,T,H,d_k]; v [B,T,H,d_v]; alpha and erase (b) [B,T,H,d_k] fp32;
    write (w) [B,T,H,d_v] fp32; S0 [B,H,d_k,d_v] fp32 or None.  Returns (o, S_out)."""
    with _on_stream(stream):
        B, T, H, d_k = q.shape
        d_v = v.shape[-1]
        dt = q.dtype
        _need(k, dt, (B, T, H, d_k), "k")
        _need(v, dt, (B, T, H, d_v), "v")
        _need(alpha, torch.float32, (B, T, H, d_k), "alpha")
        _need(erase, torch.float32, (B, T, H, d_k), "erase")
        _need(write, torch.float32, (B, T, H, d_v), "write")
        if S0 is not None:
            _need(S0, torch.float32, (B, H, d_k, d_v), "S0")
        if S_out is None:
            S_out = torch.empty((B, H, d_k, d_v), dtype=torch.float32, device=q.device)
        _need(S_out, torch.float32, (B, H, d_k, d_v), "S_out")
        if o is None:
            o = torch.empty((B, T, H, d_v), dtype=dt, device=q.device)
        _need(o, dt, (B, T, H, d_v), "o")
        shape = GdnShape(B, T, H, d_k, d_v, chunk)
        ws, nbytes = _workspace(lib().gdn_workspace_size(ctypes.byref(shape)), workspace, q.device)
        rc = lib().gdn2_chunk_forward(ctypes.byref(shape), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(alpha), _ptr(erase), _ptr(write), _ptr(S0), _ptr(S_out),
                                      _ptr(o), _ptr(ws), nbytes, _stream(stream))
        check("gdn2_chunk_forward", rc)
        return o, S_out


# ---------------------------------------------------------------------------
# Sparse State Expansion
# ---------------------------------------------------------------------------
def sse_forward(gate_logits, q, k, v, lam, S, topk, q_sh=None, k_sh=None, o=None, sel=None,
                e_sel=None, chunk=64, workspace=None, stream=None, masking=False):
    """gate_logits [B,T,H,N] fp32; q, k [B,T,H,c]; v [B,T,H,d]; lam [B,T,H,c] fp32;
    S [B,H,N+1,c,d] fp32 updated in place.  Returns o [B,T,H,d].
    masking=True calls sse_forward_masking (every partition steps over every
    token, unselected ones masked) instead of the grouped visits."""
    with _on_stream(stream):
        B, T, H, N = gate_logits.shape
        c, d = q.shape[-1], v.shape[-1]
        dt = q.dtype
        _need(gate_logits, torch.float32, (B, T, H, N), "gate_logits")
        _need(q, dt, (B, T, H, c), "q")
        _need(k, dt, (B, T, H, c), "k")
        _need(v, dt, (B, T, H, d), "v")
        _need(lam, torch.float32, (B, T, H, c), "lam")
        _need(S, torch.float32, (B, H, N + 1, c, d), "S")
        if q_sh is not None:
            _need(q_sh, dt, (B, T, H, c), "q_sh")
        if k_sh is not None:
            _need(k_sh, dt, (B, T, H, c), "k_sh")
        if o is None:
            o = torch.empty((B, T, H, d), dtype=dt, device=q.device)
        _need(o, dt, (B, T, H, d), "o")
        if sel is not None:
            _need(sel, torch.int32, (B, T, H, topk), "sel")
        if e_sel is not None:
            _need(e_sel, torch.float32, (B, T, H, topk), "e_sel")
        shape = SseShape(B, T, H, N, topk, c, d, chunk)
        ws, nbytes = _workspace(lib().sse_workspace_size(ctypes.byref(shape)), workspace, q.device)
        name = "sse_forward_masking" if masking else "sse_forward"
        rc = getattr(lib(), name)(ctypes.byref(shape), _dtype_code(q), _ptr(gate_logits), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(lam), _ptr(q_sh), _ptr(k_sh), _ptr(S),
                                  _ptr(o), _ptr(sel), _ptr(e_sel), _ptr(ws), nbytes, _stream(stream))
        check(name, rc)
        return o


def sse_decode_step(gate_logits, q, k, v, lam, S, topk, q_sh=None, k_sh=None, o=None, sel=None,
                    e_sel=None, stream=None):
    """One token per sequence: gate_logits [B,H,N] fp32; q, k [B,H,c]; v [B,H,d];
    lam [B,H,c] fp32; S [B,H,N+1,c,d] fp32 updated in place (only the selected and
    the shared states).  Returns o [B,H,d]."""
    with _on_stream(stream):
        B, H, N = gate_logits.shape
        c, d = q.shape[-1], v.shape[-1]
        dt = q.dtype
        _need(gate_logits, torch.float32, (B, H, N), "gate_logits")
        _need(q, dt, (B, H, c), "q")
        _need(k, dt, (B, H, c), "k")
        _need(v, dt, (B, H, d), "v")
        _need(lam, torch.float32, (B, H, c), "lam")
        _need(S, torch.float32, (B, H, N + 1, c, d), "S")
        if q_sh is not None:
            _need(q_sh, dt, (B, H, c), "q_sh")
        if k_sh is not None:
            _need(k_sh, dt, (B, H, c), "k_sh")
        if o is None:
            o = torch.empty((B, H, d), dtype=dt, device=q.device)
        _need(o, dt, (B, H, d), "o")
        if sel is not None:
            _need(sel, torch.int32, (B, H, topk), "sel")
        if e_sel is not None:
            _need(e_sel, torch.float32, (B, H, topk), "e_sel")
        shape = SseShape(B, 1, H, N, topk, c, d, 64)
        rc = lib().sse_decode_step(ctypes.byref(shape), _dtype_code(q), _ptr(gate_logits), _ptr(q),
                                   _ptr(k), _ptr(v), _ptr(lam), _ptr(q_sh), _ptr(k_sh), _ptr(S),
                                   _ptr(o), _ptr(sel), _ptr(e_sel), _stream(stream))
        check("sse_decode_step", rc)
        return o
