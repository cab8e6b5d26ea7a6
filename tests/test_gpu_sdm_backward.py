"""GPU parity of the SDM training path (forward keeping pre-write rows, backward
by undoing writes, addressing-softmax backward) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from sparse_state_linear_product_amd import workloads as wl
from tests.helpers import TOL_BF16, TOL_FP32, announce, maxrel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cfg(B, T, H, sqrtN, d_v, k, W, R, dtype, seed):
    return wl.SdmConfig("bwd", B, T, H, sqrtN, d_v, k, k, W, R, dtype, seed)


def _upstream(cfg, T, seed, scale_dM=1.0):
    g = torch.Generator().manual_seed(seed)
    dy = torch.randn((cfg.B, T, cfg.H, cfg.d_v), generator=g).to(cfg.dtype)
    dM = torch.randn((cfg.B, cfg.H, cfg.N, cfg.d_v), generator=g) * scale_dM
    M0 = torch.randn((cfg.B, cfg.H, cfg.N, cfg.d_v), generator=g) * 0.5
    return dy, dM, M0


def _gpu_train(x, cfg, M0, dy, dM, mode):
    import sparse_state_linear_product_amd as sslp
    xd = {k: v.to(DEV) for k, v in x.items()}
    M = M0.clone().to(DEV)
    y, ctx = sslp.sdm_forward_train(xd["sw1"], xd["sw2"], xd["sr1"], xd["sr2"], xd["v"],
                                    xd["alpha"], xd["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R,
                                    residual_mode=mode)
    M_T = M.clone()
    g = sslp.sdm_backward(ctx, xd["v"], xd["alpha"], xd["beta"], M, dy.to(DEV),
                          dM.clone().to(DEV), residual_mode=mode)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in g.items()}
    out.update(y=y.cpu(), M_T=M_T.cpu(), M_restored=M.cpu(),
               idx_w=ctx["idx_w"].cpu().numpy(), idx_r=ctx["idx_r"].cpu().numpy())
    return out


def _compare(got, ref, keys, tol, tag):
    for k_got, k_ref in keys:
        e = maxrel(got[k_got].double().numpy(), ref[k_ref], name=k_got)
        print(f"  {tag} {k_got}: {e:.2e}", flush=True)
        assert e <= tol, f"{tag} {k_got}: {e}"


GRAD_KEYS = [("dv", "dv"), ("dalpha", "dalpha"), ("dbeta", "dbeta"), ("dwt_w", "dwt_w"),
             ("dwt_r", "dwt_r"), ("dM", "dM0"), ("dsw1", "dsw1"), ("dsw2", "dsw2"),
             ("dsr1", "dsr1"), ("dsr2", "dsr2")]


def _check_full(cfg, mode, tol):
    x = wl.sdm_inputs(cfg)
    dy, dM, M0 = _upstream(cfg, cfg.T, cfg.seed + 1)
    got = _gpu_train(x, cfg, M0, dy, dM, mode)
    n = {k: wl.to_numpy_f32(v) for k, v in x.items()}
    ref_f = oracle.sdm_forward(n["sw1"], n["sw2"], n["sr1"], n["sr2"], n["v"], n["alpha"],
                               n["beta"], M0.double().numpy(), cfg.k_w, cfg.k_r, cfg.W, cfg.R,
                               residual_mode=mode)
    np.testing.assert_array_equal(got["idx_w"], ref_f["idx_w"])
    np.testing.assert_array_equal(got["idx_r"], ref_f["idx_r"])
    assert maxrel(got["y"].double().numpy(), ref_f["y"], name="y") <= tol
    # every write undone: the table is back to M0, bit for bit
    assert torch.equal(got["M_restored"], M0)
    ref = oracle.sdm_backward(n["sw1"], n["sw2"], n["sr1"], n["sr2"], n["v"], n["alpha"],
                              n["beta"], M0.double().numpy(), cfg.k_w, cfg.k_r, cfg.W, cfg.R,
                              wl.to_numpy_f32(dy).astype(np.float64), dM.double().numpy(),
                              residual_mode=mode)
    _compare(got, ref, GRAD_KEYS, tol, f"mode {mode}")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T", [1, 37])
def test_sdm_train_fp32_matches_oracle(mode, T):
    announce(f"sdm_forward_train + sdm_backward fp32 mode={mode} T={T}")
    # d_v = 40: two full 16-column slices and a ragged one of 8
    _check_full(_cfg(2, T, 2, 16, 40, 8, 32, 32, torch.float32, 500 + T + mode), mode, TOL_FP32)


def test_sdm_train_bf16_matches_oracle():
    announce("sdm_forward_train + sdm_backward bf16")
    _check_full(_cfg(1, 50, 2, 24, 64, 8, 32, 32, torch.bfloat16, 541), 0, TOL_BF16)


def test_sdm_train_budget_shapes():
    # W, R up to 64 (16 rows per lane), small d_v, unequal budgets
    announce("sdm train W=64 R=8 d_v=4 and W=5 R=48")
    _check_full(_cfg(1, 20, 1, 16, 4, 8, 64, 8, torch.float32, 551), 0, TOL_FP32)
    _check_full(_cfg(1, 20, 2, 16, 20, 8, 5, 48, torch.float32, 552), 1, TOL_FP32)


CHUNK_TRAIN = [
    # B, T, H, sqrtN, d_v, k, W = R, dtype, mode: T >= 64 and W = R = 32 or 64, so
    # the training forward runs chunk-parallel (16- or 8-token chunks).  Tables
    # of 144 and 400 slots: most slots are visited by several tokens of a chunk,
    # so later visits' pre-write rows come from the walk over the slot's visits
    (1, 100, 2, 12, 24, 8, 32, "f32", 0),
    (2, 67, 1, 12, 16, 8, 32, "f32", 1),
    (1, 72, 2, 12, 24, 8, 64, "f32", 0),
    (1, 81, 1, 20, 32, 10, 64, "f32", 1),
    (1, 80, 2, 20, 40, 8, 32, "bf16", 0),
]


@pytest.mark.parametrize("case", CHUNK_TRAIN)
def test_sdm_train_chunk_path(case):
    import sparse_state_linear_product_amd as sslp
    B, T, H, sq, dv, k, W, dt, mode = case
    dtype = torch.float32 if dt == "f32" else torch.bfloat16
    cfg = _cfg(B, T, H, sq, dv, k, W, W, dtype, 610 + sum(case[:7]) + mode)
    announce(f"sdm_forward_train chunk path {case}")
    tol = TOL_FP32 if dt == "f32" else TOL_BF16
    # gradients, the forward read and the restored table
    _check_full(cfg, mode, tol)
    # the pre-write rows against the oracle's table after each prefix
    x = wl.sdm_inputs(cfg)
    _, _, M0 = _upstream(cfg, T, cfg.seed + 1)
    xd = {kk: v.to(DEV) for kk, v in x.items()}
    M = M0.clone().to(DEV)
    _, ctx = sslp.sdm_forward_train(xd["sw1"], xd["sw2"], xd["sr1"], xd["sr2"], xd["v"],
                                    xd["alpha"], xd["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R,
                                    residual_mode=mode)
    torch.cuda.synchronize()
    saved = ctx["saved"].cpu().double().numpy()
    n = {kk: wl.to_numpy_f32(v) for kk, v in x.items()}
    iw, ww = oracle.sdm_address(n["sw1"], n["sw2"], cfg.k_w, cfg.W)
    ir, wr = oracle.sdm_address(n["sr1"], n["sr2"], cfg.k_r, cfg.R)
    ref = np.empty_like(saved)
    for t in range(T):
        Mt, _ = oracle.sdm_recurrence(iw[:, :t], ww[:, :t], ir[:, :t], wr[:, :t], n["v"][:, :t],
                                      n["alpha"][:, :t], n["beta"][:, :t], M0.double().numpy(),
                                      residual_mode=mode)
        for b in range(B):
            for h in range(H):
                ref[b, t, h] = Mt[b, h, iw[b, t, h]]
    e = maxrel(saved, ref, name="saved")
    print(f"  saved: {e:.2e}", flush=True)
    assert e <= TOL_FP32, f"saved rows: {e}"


@pytest.mark.parametrize("W", [32, 64, 9])
def test_backward_out_of_range_slot_is_contained_and_reported(W):
    # sdm_backward with a caller index outside [0, N): W = 32, 64 take the
    # chunk-parallel backward, W = 9 the per-token sweep.  The table and its
    # gradient are slices of larger buffers whose guard regions must stay
    # bitwise; the device error flag reports the call; gradients stay finite.
    import sparse_state_linear_product_amd as sslp
    announce(f"sdm_backward with an out-of-range slot, W = R = {W}")
    assert not sslp.device_error()
    B, T, H, sq, dv = 1, 80, 2, 16, 16
    N = sq * sq
    g = torch.Generator().manual_seed(95 + W)
    idx = torch.stack([torch.randperm(N, generator=g)[:W] for _ in range(B * T * H)]).int()
    idx = idx.view(B, T, H, W).contiguous()
    wt = torch.full((B, T, H, W), 1.0 / W)
    v = torch.randn((B, T, H, dv), generator=g)
    alpha = torch.full((B, T, H), 0.95)
    beta = torch.full((B, T, H), 0.5)
    dy = torch.randn((B, T, H, dv), generator=g)
    t = lambda x: x.to(DEV)
    M = torch.randn((B, H, N, dv), generator=g).to(DEV)
    _, saved = sslp.sdm_sparse_update_train(t(idx), t(wt), t(idx), t(wt), t(v), t(alpha),
                                            t(beta), M)
    torch.cuda.synchronize()
    assert not sslp.device_error()
    bad = idx.clone()
    bad[0, 70, 1, 3] = N + 5   # a bad write slot
    bad_r = idx.clone()
    bad_r[0, 10, 0, 0] = -7    # a bad read slot
    guard = 1 << 16
    n = B * H * N * dv
    mbuf = torch.randn((2 * guard + n,), generator=g).to(DEV)
    gbuf = torch.randn((2 * guard + n,), generator=g).to(DEV)
    mbuf[guard:guard + n] = M.reshape(-1)
    m0, g0 = mbuf.clone(), gbuf.clone()
    Mv = mbuf[guard:guard + n].view(B, H, N, dv)
    Gv = gbuf[guard:guard + n].view(B, H, N, dv)
    ctx = dict(idx_w=t(bad), wt_w=t(wt), idx_r=t(bad_r), wt_r=t(wt), saved=saved)
    out = sslp.sdm_backward(ctx, t(v), t(alpha), t(beta), Mv, t(dy), Gv, score_grads=False)
    torch.cuda.synchronize()
    assert sslp.device_error()
    assert not sslp.device_error()  # the query cleared it
    for buf, ref in ((mbuf, m0), (gbuf, g0)):
        assert torch.equal(buf[:guard], ref[:guard]) and torch.equal(buf[-guard:], ref[-guard:])
    for k in ("dv", "dalpha", "dbeta", "dwt_w", "dwt_r"):
        assert torch.isfinite(out[k]).all(), k


@pytest.mark.parametrize("mode", [0, 1])
def test_sdm_recurrence_backward_signed_weights(mode):
    # the recurrence alone with raw signed weights and distinct slots, read and
    # write sets overlapping within tokens
    import sparse_state_linear_product_amd as sslp
    announce(f"sdm_sparse_update_train + sdm_backward, signed weights, mode={mode}")
    rng = np.random.default_rng(560 + mode)
    B, T, H, N, dv, W, R = 1, 30, 2, 64, 24, 12, 10
    perm = np.stack([rng.permutation(N)[:W + R] for _ in range(B * T * H)])
    idx_w = perm[:, :W].reshape(B, T, H, W).astype(np.int32)
    # half the read slots are also written by the same token
    idx_r = np.concatenate([perm[:, :R // 2], perm[:, W:W + R - R // 2]], 1)
    idx_r = idx_r.reshape(B, T, H, R).astype(np.int32)
    wt_w = (rng.standard_normal((B, T, H, W)) * 0.4).astype(np.float32)
    wt_r = rng.standard_normal((B, T, H, R)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    alpha = rng.uniform(0.7, 1.0, (B, T, H)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, T, H)).astype(np.float32)
    M0 = rng.standard_normal((B, H, N, dv)).astype(np.float32)
    dy = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    dM = rng.standard_normal((B, H, N, dv)).astype(np.float32)
    t = lambda a: torch.from_numpy(a).to(DEV)
    M = t(M0).clone()
    y, saved = sslp.sdm_sparse_update_train(t(idx_w), t(wt_w), t(idx_r), t(wt_r), t(v), t(alpha),
                                            t(beta), M, residual_mode=mode)
    ctx = dict(idx_w=t(idx_w), wt_w=t(wt_w), idx_r=t(idx_r), wt_r=t(wt_r), saved=saved)
    g = sslp.sdm_backward(ctx, t(v), t(alpha), t(beta), M, t(dy), t(dM).clone(),
                          residual_mode=mode, score_grads=False)
    torch.cuda.synchronize()
    assert "dsw1" not in g
    assert torch.equal(M.cpu(), torch.from_numpy(M0))
    ref = oracle.sdm_recurrence_backward(idx_w, wt_w, idx_r, wt_r, v, alpha, beta,
                                         M0.astype(np.float64), dy.astype(np.float64),
                                         dM.astype(np.float64), residual_mode=mode)
    got = {k: v.cpu() for k, v in g.items()}
    _compare(got, ref, GRAD_KEYS[:6], TOL_FP32, f"signed mode {mode}")


def test_sdm_backward_empty_sequence():
    import sparse_state_linear_product_amd as sslp
    announce("sdm_backward T=0")
    B, H, N, dv, W, R = 1, 1, 16, 8, 4, 4
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt, device=DEV)
    ctx = dict(idx_w=z(B, 0, H, W, dt=torch.int32), wt_w=z(B, 0, H, W),
               idx_r=z(B, 0, H, R, dt=torch.int32), wt_r=z(B, 0, H, R), saved=z(B, 0, H, W, dv))
    M = torch.randn((B, H, N, dv), device=DEV)
    dM = torch.randn((B, H, N, dv), device=DEV)
    M_in, dM_in = M.clone(), dM.clone()
    g = sslp.sdm_backward(ctx, z(B, 0, H, dv), z(B, 0, H), z(B, 0, H), M, z(B, 0, H, dv), dM)
    torch.cuda.synchronize()
    assert torch.equal(M, M_in) and torch.equal(g["dM"], dM_in)


def test_sdm_train_full_size_prefix_gradients():
    # the 1.4B prefill layer (B=1, T=8192, H=2, N=57600, d_v=960, k=W=R=32) in
    # the launch configuration the benchmark times.  With dy zero after the
    # first 64 tokens and no final-table gradient, nothing flows back from the
    # later tokens (every gradient there is exactly zero), so the first 64
    # tokens' gradients equal those of the 64-token problem, which the oracle
    # computes; the table must come back to M0 bit for bit.
    import sparse_state_linear_product_amd as sslp
    cfg = wl.SDM_14B
    Tp = 64
    announce(f"{cfg.name} training forward + backward, prefix {Tp} checked")
    x = wl.sdm_inputs(cfg)
    xd = {k: v.to(DEV) for k, v in x.items()}
    g0 = torch.Generator(device=DEV).manual_seed(cfg.seed + 5)
    M = torch.randn((cfg.B, cfg.H, cfg.N, cfg.d_v), generator=g0, device=DEV) * 0.1
    M0 = M.clone()
    dy = torch.zeros((cfg.B, cfg.T, cfg.H, cfg.d_v), dtype=cfg.dtype, device=DEV)
    dy[:, :Tp] = torch.randn((cfg.B, Tp, cfg.H, cfg.d_v), generator=g0, device=DEV).to(cfg.dtype)
    y, ctx = sslp.sdm_forward_train(xd["sw1"], xd["sw2"], xd["sr1"], xd["sr2"], xd["v"],
                                    xd["alpha"], xd["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R)
    g = sslp.sdm_backward(ctx, xd["v"], xd["alpha"], xd["beta"], M, dy)
    torch.cuda.synchronize()
    assert torch.equal(M, M0)
    for k in ("dv", "dalpha", "dbeta", "dwt_w", "dwt_r", "dsw1", "dsw2", "dsr1", "dsr2"):
        assert not torch.any(g[k][:, Tp:] != 0), k
    n = {k: wl.to_numpy_f32(v[:, :Tp]) for k, v in x.items()}
    ref = oracle.sdm_backward(n["sw1"], n["sw2"], n["sr1"], n["sr2"], n["v"], n["alpha"],
                              n["beta"], M0.double().cpu().numpy(), cfg.k_w, cfg.k_r, cfg.W,
                              cfg.R, dy[:, :Tp].double().cpu().numpy())
    got = {k: (v[:, :Tp] if k != "dM" else v).cpu() for k, v in g.items()}
    _compare(got, ref, GRAD_KEYS, TOL_BF16, "full-size prefix")
