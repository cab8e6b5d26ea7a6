"""sdm_forward_noalloc (fixed per-GPU scratch, no allocation) against sdm_forward
(caller workspace), through the C ABI: identical kernels, so identical results,
on two calls in a row of which the second is smaller."""
import pytest

from sparse_state_linear_product_amd import workloads as wl
from tests.helpers import announce

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # B, T, H, sqrtN, d_v, k_w, k_r, W, R, dtype: the chunk-parallel path (W = R = 32,
    # T >= 64, chunk plans in the scratch), then a smaller per-token-path case
    (1, 300, 2, 240, 64, 32, 32, 32, 32, torch.bfloat16),
    (2, 70, 1, 16, 24, 8, 6, 9, 7, torch.float32),
]


def _inputs(case, seed):
    B, T, H, sq, dv, kw, kr, W, R, dt = case
    cfg = wl.SdmConfig("noalloc", B, T, H, sq, dv, kw, kr, W, R, dt, seed)
    x = {k: v.to(DEV) for k, v in wl.sdm_inputs(cfg).items()}
    M0 = torch.randn((B, H, sq * sq, dv), generator=torch.Generator().manual_seed(seed)).to(DEV)
    return cfg, x, M0


def _run(fn, cfg, x, M0, **kw):
    M = M0.clone()
    shp = (cfg.B, cfg.T, cfg.H)
    y = torch.empty(shp + (cfg.d_v,), dtype=cfg.dtype, device=DEV)
    iw = torch.empty(shp + (cfg.W,), dtype=torch.int32, device=DEV)
    ir = torch.empty(shp + (cfg.R,), dtype=torch.int32, device=DEV)
    fn(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"], x["beta"], M, y=y,
       k_w=cfg.k_w, k_r=cfg.k_r, W=cfg.W, R=cfg.R, idx_w=iw, idx_r=ir, **kw)
    return y, M, iw, ir


def test_noalloc_matches_sdm_forward_on_consecutive_calls():
    import sparse_state_linear_product_amd as sslp

    for n, case in enumerate(CASES):
        announce(f"sdm_forward_noalloc call {n + 1}: {case}")
        cfg, x, M0 = _inputs(case, 900 + n)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        got = _run(sslp.sdm_forward_noalloc, cfg, x, M0)
        torch.cuda.synchronize()
        # the call itself allocates nothing (M0.clone() and the outputs come first)
        blocks = sum(-(-t.numel() * t.element_size() // 512) * 512 for t in got)
        assert torch.cuda.memory_allocated() - before == blocks
        ref = _run(sslp.sdm_forward, cfg, x, M0)
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "M", "idx_w", "idx_r"), got, ref):
            assert torch.equal(a, b), f"call {n + 1}: {name} differs from sdm_forward"
        print(f"  call {n + 1}: y, M, idx_w, idx_r bitwise equal to sdm_forward", flush=True)
        del got, ref, x, M0
