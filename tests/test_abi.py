"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before touching HIP."""
import ctypes
import os
import re

import pytest

from sparse_state_linear_product_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sslp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|void)\s*\*?\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("sdm_forward", "sdm_decode_step", "sse_forward", "sse_forward_masking",
                     "sse_decode_step",
                     "gdn_chunk_forward",
                     "sdm_address", "sdm_sparse_update", "sslp_last_error", "sslp_version"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"missing exports: {missing}"
    assert set(_lib.SIGNATURES) >= set(declared_functions())
    assert lib.sslp_version() == 1


def _sdm(B=1, T=4, H=1, sqrtN=8, d_v=16, k_w=4, k_r=4, W=4, R=4):
    return _lib.SdmShape(B, T, H, sqrtN, d_v, k_w, k_r, W, R)


FAKE = ctypes.c_void_p(0x1000)  # aligned non-NULL pointer; never dereferenced (rejected first)
MISALIGNED = ctypes.c_void_p(0x1004)


def _fwd(shape, dtype=0, mode=0, ptrs=None, ws_bytes=1 << 20):
    ptrs = ptrs or [FAKE] * 9 + [None] * 4 + [FAKE]
    return _lib.lib().sdm_forward(ctypes.byref(shape), dtype, mode, *ptrs, ws_bytes, None)


@pytest.mark.parametrize("shape,code,msg", [
    (_sdm(W=20), _lib.SSLP_ERR_INVALID_ARG, "W=20 > k_w^2"),
    (_sdm(k_w=9), _lib.SSLP_ERR_INVALID_ARG, "k_w, k_r must be <= sqrtN"),
    (_sdm(B=0), _lib.SSLP_ERR_INVALID_ARG, "B, H must be >= 1"),
    (_sdm(T=-1), _lib.SSLP_ERR_INVALID_ARG, "B, H must be >= 1"),
    (_sdm(d_v=6), _lib.SSLP_ERR_UNSUPPORTED, "multiple of 4"),
    (_sdm(sqrtN=2000, k_w=4, k_r=4), _lib.SSLP_ERR_UNSUPPORTED, "sqrtN 2000"),
    (_sdm(sqrtN=100, k_w=80, k_r=4), _lib.SSLP_ERR_UNSUPPORTED, "<= 64"),
    (_sdm(sqrtN=100, k_w=20, k_r=20, W=200), _lib.SSLP_ERR_UNSUPPORTED, "<= 128"),
])
def test_sdm_forward_shape_errors(shape, code, msg):
    assert _fwd(shape) == code
    assert msg in _lib.lib().sslp_last_error().decode()


def test_sdm_forward_pointer_errors():
    lib = _lib.lib()
    ptrs = [FAKE] * 9 + [None] * 4 + [FAKE]
    for i, name in enumerate(["sw1", "sw2", "sr1", "sr2", "v", "alpha", "beta", "M", "y"]):
        p = list(ptrs)
        p[i] = None
        assert _fwd(_sdm(), ptrs=p) == _lib.SSLP_ERR_INVALID_ARG
        assert f"{name} must not be NULL" in lib.sslp_last_error().decode()
        p[i] = MISALIGNED
        assert _fwd(_sdm(), ptrs=p) == _lib.SSLP_ERR_INVALID_ARG
        assert "aligned" in lib.sslp_last_error().decode()


def test_sdm_forward_workspace_and_flags():
    lib = _lib.lib()
    s = _sdm()
    need = lib.sdm_workspace_size(ctypes.byref(s))
    assert need > 0
    assert _fwd(s, ws_bytes=need - 1) == _lib.SSLP_ERR_WORKSPACE
    assert _fwd(s, dtype=7) == _lib.SSLP_ERR_INVALID_ARG
    assert _fwd(s, mode=2) == _lib.SSLP_ERR_INVALID_ARG
    assert lib.sdm_workspace_size(ctypes.byref(_sdm(W=65))) == 0  # W > N


@pytest.mark.parametrize("W,k,chunk", [(32, 6, 16), (64, 8, 8), (40, 7, None)])
def test_sdm_workspace_holds_the_chunk_plans(W, k, chunk):
    # W = R = 32 and W = R = 64 with T >= 64 take the chunk-parallel recurrence
    # (chunks of 16 and 8 tokens), whose per-chunk plans (7680 words each) live
    # in the workspace after the addressing; other shapes need the addressing only
    lib = _lib.lib()

    def a256(x):
        return (x + 255) // 256 * 256

    for T in (63, 100):
        s = _sdm(B=2, T=T, H=3, sqrtN=16, d_v=16, k_w=k, k_r=k, W=W, R=W)
        addressing = 4 * a256(2 * T * 3 * W * 4)
        plans = 0 if chunk is None or T < 64 else a256(2 * 3 * -(-T // chunk) * 7680 * 4)
        assert lib.sdm_workspace_size(ctypes.byref(s)) == addressing + plans, (W, T)


def test_sdm_decode_requires_single_token():
    lib = _lib.lib()
    s = _sdm(T=3)
    rc = lib.sdm_decode_step(ctypes.byref(s), 0, 0, *([FAKE] * 9 + [None] * 4 + [FAKE]), 1 << 20,
                             None)
    assert rc == _lib.SSLP_ERR_INVALID_ARG and "T == 1" in lib.sslp_last_error().decode()


def test_sdm_training_entry_errors():
    # argument checks of the training forward and the backward (no GPU call is made)
    lib = _lib.lib()
    s = _sdm()
    # sdm_forward_train needs the addressing outputs and the saved rows
    assert lib.sdm_forward_train(ctypes.byref(s), 0, 0, *([FAKE] * 13), None, None, 0, None) == \
        _lib.SSLP_ERR_INVALID_ARG
    assert "saved" in lib.sslp_last_error().decode()
    assert lib.sdm_forward_train(ctypes.byref(s), 0, 0, *([FAKE] * 9), None, *([FAKE] * 4),
                                 None, 0, None) == _lib.SSLP_ERR_INVALID_ARG
    assert lib.sdm_sparse_update_train(ctypes.byref(s), 0, 3, *([FAKE] * 10), None, 0, None) == \
        _lib.SSLP_ERR_INVALID_ARG
    # a shape on the chunk-parallel path needs its plans: short or misaligned
    # workspaces are refused before any launch
    assert lib.sdm_train_workspace_size(ctypes.byref(s)) == 0  # per-token shape
    c = _sdm(T=64, sqrtN=16, k_w=6, k_r=6, W=32, R=32)
    need = lib.sdm_train_workspace_size(ctypes.byref(c))
    assert need == 4 * 7680 * 4  # B = H = 1: 4 chunks of 7,680 words
    assert lib.sdm_forward_train(ctypes.byref(c), 0, 0, *([FAKE] * 14), FAKE, need - 1, None) == \
        _lib.SSLP_ERR_WORKSPACE
    assert lib.sdm_sparse_update_train(ctypes.byref(c), 0, 0, *([FAKE] * 10), None, need,
                                       None) == _lib.SSLP_ERR_WORKSPACE
    assert lib.sdm_sparse_update_train(ctypes.byref(c), 0, 0, *([FAKE] * 10), MISALIGNED, need,
                                       None) == _lib.SSLP_ERR_INVALID_ARG
    need = lib.sdm_backward_workspace_size(ctypes.byref(s))
    assert need > 0
    ptrs = [FAKE] * 20
    assert lib.sdm_backward(ctypes.byref(s), 0, 0, *ptrs, FAKE, need - 1, None) == \
        _lib.SSLP_ERR_WORKSPACE
    assert lib.sdm_backward(ctypes.byref(s), 0, 0, *ptrs, None, need, None) == \
        _lib.SSLP_ERR_WORKSPACE
    half = ptrs[:17] + [None] + ptrs[18:]  # dsw1 given, dsw2 NULL
    assert lib.sdm_backward(ctypes.byref(s), 0, 0, *half, FAKE, need, None) == \
        _lib.SSLP_ERR_INVALID_ARG
    assert "pairs" in lib.sslp_last_error().decode()
    no_dy = ptrs[:9] + [None] + ptrs[10:]
    assert lib.sdm_backward(ctypes.byref(s), 0, 0, *no_dy, FAKE, need, None) == \
        _lib.SSLP_ERR_INVALID_ARG
    assert "dy" in lib.sslp_last_error().decode()


def test_norm_gate_errors():
    lib = _lib.lib()
    ng = lib.sdm_norm_gate
    assert ng(4, 6, 0, FAKE, FAKE, FAKE, 1e-6, 1, FAKE, None) == _lib.SSLP_ERR_UNSUPPORTED
    assert ng(4, 8, 0, FAKE, FAKE, FAKE, 1e-6, 3, FAKE, None) == _lib.SSLP_ERR_INVALID_ARG
    assert ng(4, 8, 0, FAKE, None, FAKE, 1e-6, 1, FAKE, None) == _lib.SSLP_ERR_INVALID_ARG
    assert "gate" in lib.sslp_last_error().decode()
    assert ng(4, 8, 0, FAKE, FAKE, FAKE, -1.0, 1, FAKE, None) == _lib.SSLP_ERR_INVALID_ARG
    assert ng(4, 8, 2, FAKE, FAKE, FAKE, 1e-6, 1, FAKE, None) == _lib.SSLP_ERR_INVALID_ARG
    assert ng(0, 8, 0, None, None, None, 1e-6, 1, None, None) == _lib.SSLP_OK


def test_sdm_address_errors():
    lib = _lib.lib()
    s = _sdm()
    assert lib.sdm_address(ctypes.byref(s), 0, FAKE, FAKE, 9, 4, FAKE, FAKE, None) == \
        _lib.SSLP_ERR_INVALID_ARG
    assert lib.sdm_address(ctypes.byref(s), 0, FAKE, FAKE, 4, 17, FAKE, FAKE, None) == \
        _lib.SSLP_ERR_INVALID_ARG
    assert lib.sdm_address(ctypes.byref(s), 0, None, FAKE, 4, 4, FAKE, FAKE, None) == \
        _lib.SSLP_ERR_INVALID_ARG


def test_gdn_and_sse_shape_errors():
    lib = _lib.lib()
    g = _lib.GdnShape(1, 8, 1, 64, 128, 64)
    assert lib.gdn_chunk_forward(ctypes.byref(g), 1, 0, *([FAKE] * 9), 0, None) == \
        _lib.SSLP_ERR_UNSUPPORTED
    g = _lib.GdnShape(1, 8, 1, 128, 128, 64)
    assert lib.gdn_chunk_forward(ctypes.byref(g), 1, 5, *([FAKE] * 9), 0, None) == \
        _lib.SSLP_ERR_INVALID_ARG
    g = _lib.GdnShape(1, 8, 1, 128, 128, 64)
    assert lib.gdn2_chunk_forward(ctypes.byref(g), 0, *([FAKE] * 10), 0, None) == \
        _lib.SSLP_ERR_UNSUPPORTED
    assert lib.gdn2_chunk_forward(ctypes.byref(g), 1, *([FAKE] * 9), None, 0, None) == \
        _lib.SSLP_ERR_WORKSPACE
    assert lib.gdn2_chunk_forward(ctypes.byref(g), 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, 1 << 30, None) == _lib.SSLP_ERR_INVALID_ARG
    s = _lib.SseShape(1, 8, 1, 8, 9, 128, 128, 64)
    assert lib.sse_forward(ctypes.byref(s), 1, *([FAKE] * 12), 0, None) == _lib.SSLP_ERR_INVALID_ARG
    s = _lib.SseShape(1, 8, 1, 8, 2, 64, 128, 64)
    assert lib.sse_forward(ctypes.byref(s), 1, *([FAKE] * 12), 0, None) == _lib.SSLP_ERR_UNSUPPORTED
    # the masking execution validates exactly like the grouped one
    assert lib.sse_forward_masking(ctypes.byref(s), 1, *([FAKE] * 12), 0, None) == \
        _lib.SSLP_ERR_UNSUPPORTED
    s = _lib.SseShape(1, 8, 1, 8, 9, 128, 128, 64)
    assert lib.sse_forward_masking(ctypes.byref(s), 1, *([FAKE] * 12), 0, None) == \
        _lib.SSLP_ERR_INVALID_ARG
    s = _lib.SseShape(1, 8, 1, 8, 2, 128, 128, 64)
    assert lib.sse_forward_masking(ctypes.byref(s), 0, *([FAKE] * 12), 0, None) == \
        _lib.SSLP_ERR_UNSUPPORTED
    assert b"sse_forward_masking" in lib.sslp_last_error()
    # the grouped execution needs its workspace (visit lists, contributions by
    # slot) even when the caller takes the routing
    s = _lib.SseShape(1, 8, 1, 8, 2, 128, 128, 64)
    assert lib.sse_workspace_size(ctypes.byref(s)) >= 8 * 3 * 128 * 2
    assert lib.sse_forward(ctypes.byref(s), 1, *([FAKE] * 12), 0, None) == _lib.SSLP_ERR_WORKSPACE
    # the decode step takes exactly one token per sequence
    s = _lib.SseShape(2, 2, 1, 8, 2, 128, 128, 64)
    assert lib.sse_decode_step(ctypes.byref(s), 1, *([FAKE] * 11), None) == _lib.SSLP_ERR_INVALID_ARG
    s = _lib.SseShape(2, 1, 1, 8, 9, 128, 128, 64)
    assert lib.sse_decode_step(ctypes.byref(s), 1, *([FAKE] * 11), None) == _lib.SSLP_ERR_INVALID_ARG
    s = _lib.SseShape(2, 1, 1, 8, 2, 128, 128, 64)
    assert lib.sse_decode_step(ctypes.byref(s), 0, *([FAKE] * 11), None) == _lib.SSLP_ERR_UNSUPPORTED
    assert lib.sse_decode_step(ctypes.byref(s), 1, *([None] * 11), None) == _lib.SSLP_ERR_INVALID_ARG


def test_sdm_forward_noalloc_rejects_oversize_before_any_hip_call():
    lib = _lib.lib()
    cap = lib.sdm_noalloc_scratch_bytes()
    assert cap == 64 << 20
    # a long 1.4B-layer sequence needs more chunk-plan scratch than the fixed array
    big = _sdm(B=1, T=1 << 16, H=2, sqrtN=240, d_v=960, k_w=32, k_r=32, W=32, R=32)
    need = lib.sdm_workspace_size(ctypes.byref(big))
    assert need > cap
    ptrs = [FAKE] * 9 + [None] * 4
    rc = lib.sdm_forward_noalloc(ctypes.byref(big), 1, 0, *ptrs, None)
    assert rc == _lib.SSLP_ERR_WORKSPACE
    assert "scratch" in lib.sslp_last_error().decode()
    # bad shapes are rejected as in sdm_forward
    assert lib.sdm_forward_noalloc(ctypes.byref(_sdm(W=20)), 0, 0, *ptrs, None) == \
        _lib.SSLP_ERR_INVALID_ARG
    assert lib.sdm_forward_noalloc(ctypes.byref(_sdm()), 0, 0, *([None] + ptrs[1:]), None) == \
        _lib.SSLP_ERR_INVALID_ARG
