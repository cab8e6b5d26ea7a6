"""Pins for the SDM backward oracle (undoing writes): every gradient is checked
against central finite differences of the forward oracle, which shares no code
with the backward.  A dropped term, a wrong sign or a transposed index in any of
dv, dalpha, dbeta, dwt_w, dwt_r, dM0 or the score-half gradients moves the
result far outside the finite-difference error."""
import numpy as np
import pytest

import oracle

B, T, H, SQN, DV = 1, 6, 2, 4, 3
KW, KR, W, R = 3, 3, 4, 3


def _separated_halves(rng):
    # half scores a * 0.31 and b * 0.17 (permuted per token/head, plus noise of
    # at most 0.004): the selected pairs mix several a and b, and any two
    # candidate sums differ by more than 0.01, so a perturbation of 2^-10
    # never changes a selection.  The values are multiples of 2^-12 below 2,
    # so every fp32 candidate sum, perturbed or not, is exact and the
    # differences see no rounding of the ranking key.
    s1 = np.empty((B, T, H, SQN), np.float32)
    s2 = np.empty((B, T, H, SQN), np.float32)
    for idx in np.ndindex(B, T, H):
        s1[idx] = rng.permutation(SQN) * 0.31 + rng.uniform(-0.004, 0.004, SQN)
        s2[idx] = rng.permutation(SQN) * 0.17 + rng.uniform(-0.004, 0.004, SQN)
    return np.round(s1 * 4096) / 4096, np.round(s2 * 4096) / 4096


def _problem(seed):
    rng = np.random.default_rng(seed)
    sw1, sw2 = _separated_halves(rng)
    sr1, sr2 = _separated_halves(rng)
    x = dict(sw1=sw1, sw2=sw2, sr1=sr1, sr2=sr2,
             v=rng.standard_normal((B, T, H, DV)).astype(np.float32),
             alpha=rng.uniform(0.6, 0.99, (B, T, H)).astype(np.float32),
             beta=rng.uniform(0.2, 0.9, (B, T, H)).astype(np.float32))
    M0 = rng.standard_normal((B, H, SQN * SQN, DV))
    dy = rng.standard_normal((B, T, H, DV))
    dM = rng.standard_normal((B, H, SQN * SQN, DV))
    return x, M0, dy, dM


def _loss(x, M0, dy, dM, mode):
    out = oracle.sdm_forward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"],
                             x["beta"], M0, KW, KR, W, R, residual_mode=mode)
    return float(np.sum(out["y"] * dy) + np.sum(out["M"] * dM))


def _fd_float32(x, name, M0, dy, dM, mode, h=2.0 ** -9):
    """Central differences over every entry of the float32 input `name`, divided
    by the float32 step actually taken."""
    base = x[name]
    g = np.zeros(base.shape)
    for idx in np.ndindex(base.shape):
        xp, xm = dict(x), dict(x)
        ap, am = base.copy(), base.copy()
        ap[idx] = np.float32(base[idx] + h)
        am[idx] = np.float32(base[idx] - h)
        xp[name], xm[name] = ap, am
        step = float(ap[idx]) - float(am[idx])
        g[idx] = (_loss(xp, M0, dy, dM, mode) - _loss(xm, M0, dy, dM, mode)) / step
    return g


def _close(got, fd, tag, rtol=2e-5):
    scale = max(np.abs(fd).max(), 1e-6)
    err = np.abs(got - fd).max() / scale
    assert err <= rtol, f"{tag}: max rel err {err:.3e}"


@pytest.mark.parametrize("mode", [0, 1])
def test_gate_value_and_table_gradients_match_finite_differences(mode):
    x, M0, dy, dM = _problem(11 + mode)
    g = oracle.sdm_backward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"],
                            x["beta"], M0, KW, KR, W, R, dy, dM, residual_mode=mode)
    for name, key in (("v", "dv"), ("alpha", "dalpha"), ("beta", "dbeta")):
        _close(g[key], _fd_float32(x, name, M0, dy, dM, mode), f"mode {mode} {key}")
    # M0 is float64 at the oracle's boundary and the loss is linear in it
    fd = np.zeros(M0.shape)
    for idx in np.ndindex(M0.shape):
        mp, mm = M0.copy(), M0.copy()
        mp[idx] += 0.5
        mm[idx] -= 0.5
        fd[idx] = _loss(x, mp, dy, dM, mode) - _loss(x, mm, dy, dM, mode)
    _close(g["dM0"], fd, f"mode {mode} dM0", rtol=1e-9)


@pytest.mark.parametrize("mode", [0, 1])
def test_score_half_gradients_match_finite_differences(mode):
    x, M0, dy, dM = _problem(21 + mode)
    g = oracle.sdm_backward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"],
                            x["beta"], M0, KW, KR, W, R, dy, dM, residual_mode=mode)
    for name in ("sw1", "sw2", "sr1", "sr2"):
        fd = _fd_float32(x, name, M0, dy, dM, mode, h=2.0 ** -10)
        assert np.abs(fd).max() > 1e-2, f"{name}: selections leave no gradient to check"
        _close(g["d" + name], fd, f"mode {mode} d{name}")
    # halves outside the per-half top-k get exactly zero
    idx_w, _ = oracle.sdm_address(x["sw1"], x["sw2"], KW, W)
    for b, t, h in np.ndindex(B, T, H):
        used = set((idx_w[b, t, h] // SQN).tolist())
        for a in range(SQN):
            if a not in used:
                assert g["dsw1"][b, t, h, a] == 0.0


@pytest.mark.parametrize("mode", [0, 1])
def test_weight_gradients_match_finite_differences(mode):
    # the recurrence alone, with arbitrary (unnormalised, signed) weights
    rng = np.random.default_rng(31 + mode)
    N = 10
    idx_w = np.stack([rng.permutation(N)[:W] for _ in range(B * T * H)]).reshape(B, T, H, W)
    idx_r = rng.integers(0, N, (B, T, H, R)).astype(np.int32)
    wt_w = rng.standard_normal((B, T, H, W)) * 0.5
    wt_r = rng.standard_normal((B, T, H, R))
    v = rng.standard_normal((B, T, H, DV)).astype(np.float32)
    alpha = rng.uniform(0.5, 1.0, (B, T, H)).astype(np.float32)
    beta = rng.uniform(0.1, 1.0, (B, T, H)).astype(np.float32)
    M0 = rng.standard_normal((B, H, N, DV))
    dy = rng.standard_normal((B, T, H, DV))
    dM = rng.standard_normal((B, H, N, DV))

    def loss(ww, wr):
        M, y = oracle.sdm_recurrence(idx_w, ww, idx_r, wr, v, alpha, beta, M0, mode)
        return float(np.sum(y * dy) + np.sum(M * dM))

    g = oracle.sdm_recurrence_backward(idx_w, wt_w, idx_r, wt_r, v, alpha, beta, M0, dy, dM,
                                       mode)
    h = 1e-5
    for arr, key, is_w in ((wt_w, "dwt_w", True), (wt_r, "dwt_r", False)):
        fd = np.zeros(arr.shape)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            lp = loss(ap, wt_r) if is_w else loss(wt_w, ap)
            lm = loss(am, wt_r) if is_w else loss(wt_w, am)
            fd[idx] = (lp - lm) / (2 * h)
        _close(g[key], fd, f"mode {mode} {key}", rtol=1e-7)


def test_no_write_gate_leaves_values_without_gradient():
    # beta = 0: nothing is written, so v has no influence and the table
    # gradient is the upstream one plus the reads, each decayed by nothing
    x, M0, dy, dM = _problem(41)
    x["beta"][:] = 0.0
    x["alpha"][:] = 1.0
    g = oracle.sdm_backward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"],
                            x["beta"], M0, KW, KR, W, R, dy, dM)
    assert np.all(g["dv"] == 0.0)
    out = oracle.sdm_forward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"],
                             x["beta"], M0, KW, KR, W, R)
    expect = dM.copy()
    for b, t, h in np.ndindex(B, T, H):
        for m in range(R):
            expect[b, h, out["idx_r"][b, t, h, m]] += out["wt_r"][b, t, h, m] * dy[b, t, h]
    np.testing.assert_allclose(g["dM0"], expect, rtol=0, atol=1e-12)
