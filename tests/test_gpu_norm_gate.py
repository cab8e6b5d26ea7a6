"""GPU parity of the read epilogue (RMS-Norm + output gate) against the oracle,
alone and after the SDM forward at the 1.4B prefill shape."""
import numpy as np
import pytest

import oracle
from sparse_state_linear_product_amd import workloads as wl
from tests.helpers import TOL_BF16, TOL_FP32, announce, maxrel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(rows, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    y = (torch.randn((rows, d), generator=g) * 3.0).to(dtype)
    gate = torch.randn((rows, d), generator=g).to(dtype)
    gamma = torch.rand((d,), generator=g) + 0.5
    return y, gate, gamma


@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_FP32), (torch.bfloat16, TOL_BF16)])
@pytest.mark.parametrize("act", ["none", "silu", "sigmoid"])
@pytest.mark.parametrize("rows,d", [(1, 4), (7, 40), (130, 960), (3, 1024), (3, 1028), (5, 4096)])
def test_norm_gate_matches_oracle(dtype, tol, act, rows, d):
    import sparse_state_linear_product_amd as sslp
    announce(f"sdm_norm_gate {dtype} act={act} rows={rows} d={d}")
    y, gate, gamma = _inputs(rows, d, dtype, 100 + rows + d)
    o = sslp.sdm_norm_gate(y.to(DEV), gamma.to(DEV), None if act == "none" else gate.to(DEV),
                           eps=1e-6, act=act)
    torch.cuda.synchronize()
    ref = oracle.norm_gate(wl.to_numpy_f32(y), wl.to_numpy_f32(gate), gamma.numpy(), 1e-6, act)
    e = maxrel(o.cpu().double().numpy(), ref, name="o")
    print(f"  {act} {rows}x{d}: {e:.2e}", flush=True)
    assert e <= tol


def test_norm_gate_in_place_zero_rows_and_zero_row():
    import sparse_state_linear_product_amd as sslp
    announce("sdm_norm_gate in place, rows = 0, an all-zero row")
    y, gate, gamma = _inputs(9, 64, torch.float32, 7)
    y[3] = 0.0
    ref = oracle.norm_gate(y.numpy(), gate.numpy(), gamma.numpy(), 1e-5, "silu")
    yd = y.to(DEV)
    out = sslp.sdm_norm_gate(yd, gamma.to(DEV), gate.to(DEV), eps=1e-5, act="silu", o=yd)
    torch.cuda.synchronize()
    assert out.data_ptr() == yd.data_ptr()
    assert maxrel(yd.cpu().double().numpy(), ref, name="yd") <= TOL_FP32
    assert torch.all(yd[3] == 0)
    empty = torch.empty((0, 64), device=DEV)
    assert sslp.sdm_norm_gate(empty, gamma.to(DEV), empty, act="silu").shape == (0, 64)


def test_norm_gate_after_sdm_forward_full_size():
    # the 1.4B prefill layer: read y [1,8192,2,960] bf16 from the recurrence,
    # then the epilogue in the configuration the benchmark times; sampled rows
    # are checked against the oracle applied to the GPU's own y (the epilogue's
    # input), so the check isolates this step
    import sparse_state_linear_product_amd as sslp
    cfg = wl.SDM_14B
    announce(f"{cfg.name}: sdm_forward then sdm_norm_gate")
    x = {k: v.to(DEV) for k, v in wl.sdm_inputs(cfg).items()}
    M = torch.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device=DEV)
    y = sslp.sdm_forward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"], x["beta"], M,
                         cfg.k_w, cfg.k_r, cfg.W, cfg.R)
    g = torch.Generator(device=DEV).manual_seed(cfg.seed + 9)
    gate = torch.randn(y.shape, generator=g, device=DEV).to(cfg.dtype)
    gamma = torch.rand((cfg.d_v,), generator=g, device=DEV) + 0.5
    o = sslp.sdm_norm_gate(y, gamma, gate, eps=1e-6, act="silu")
    torch.cuda.synchronize()
    rows = np.random.default_rng(3).choice(cfg.T * cfg.H, 256, replace=False)
    yf = y.reshape(-1, cfg.d_v)[torch.from_numpy(rows).to(DEV)]
    gf = gate.reshape(-1, cfg.d_v)[torch.from_numpy(rows).to(DEV)]
    ref = oracle.norm_gate(wl.to_numpy_f32(yf.cpu()), wl.to_numpy_f32(gf.cpu()),
                           gamma.cpu().numpy(), 1e-6, "silu")
    got = o.reshape(-1, cfg.d_v)[torch.from_numpy(rows).to(DEV)].cpu().double().numpy()
    assert maxrel(got, ref, name="got") <= TOL_BF16
