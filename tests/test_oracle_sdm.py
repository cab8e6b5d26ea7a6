"""Pins for the SDM oracle: printed worked examples, brute force, invariants and
the dense limit.  None of these re-types the oracle's own formula."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _two_slot_run(mode):
    g = _gold("sdm_two_slot.json")
    # sqrtN = 2, k = 2, W = R = 2.  Half 1 ties (both 0) and half 2 = [0, -10]:
    # candidates: slot0 = 0, slot1 = -10, slot2 = 0, slot3 = -10 -> top-2 = {0, 2}
    # with equal scores, hence softmax weights 0.5 / 0.5 (the example's k).
    s1 = np.array([[[[0.0, 0.0]]]], np.float32)
    s2 = np.array([[[[0.0, -10.0]]]], np.float32)
    out = {}
    M0 = np.array([[[[g["M_prev"][0]], [7.0], [g["M_prev"][1]], [9.0]]]])  # [B,H,N=4,dv=1]
    v = np.full((1, 1, 1, 1), g["v"], np.float32)
    alpha = np.full((1, 1, 1), g["alpha"], np.float32)
    beta = np.full((1, 1, 1), g["beta"], np.float32)
    out = oracle.sdm_forward(s1, s2, s1, s2, v, alpha, beta, M0, 2, 2, 2, 2, residual_mode=mode)
    return g, out, M0


def test_two_slot_example_selection():
    g, out, _ = _two_slot_run(0)
    assert out["idx_w"].ravel().tolist() == [0, 2]
    np.testing.assert_array_equal(out["wt_w"].ravel(), g["k"])


@pytest.mark.parametrize("mode,key", [(0, "expected_shared_fig2"), (1, "expected_per_slot_eq4")])
def test_two_slot_example_update(mode, key):
    g, out, M0 = _two_slot_run(mode)
    M = out["M"].reshape(-1)
    # alpha = 0.8 is not exact in binary; the printed values are exact decimals
    np.testing.assert_allclose([M[0], M[2]], g[key], rtol=0, atol=1e-6)
    # unselected slots 1 and 3 untouched, bitwise
    assert M[1] == M0.reshape(-1)[1] and M[3] == M0.reshape(-1)[3]


def test_two_slot_modes_differ():
    _, a, _ = _two_slot_run(0)
    _, b, _ = _two_slot_run(1)
    assert abs(a["M"].reshape(-1)[0] - b["M"].reshape(-1)[0]) > 0.2


def test_delta_rule_example_through_sdm():
    g = _gold("delta_rule_example.json")
    one = np.zeros((1, 1, 1, 1), np.float32)  # sqrtN = 1: the single slot, weight 1
    M0 = np.full((1, 1, 1, 1), g["prediction"])
    v = np.full((1, 1, 1, 1), g["target"], np.float32)
    out = oracle.sdm_forward(one, one, one, one, v, np.ones((1, 1, 1), np.float32),
                             np.full((1, 1, 1), g["beta"], np.float32), M0, 1, 1, 1, 1)
    assert out["wt_w"].item() == 1.0
    assert out["y"].item() == g["expected_new_prediction"]


def _brute_top(s1, s2, budget):
    """Global top-budget over ALL N = sqrtN^2 slots (every slot scored)."""
    n = s1.shape[-1]
    keys = (s1[:, None] + s2[None, :]).astype(np.float32).reshape(-1)  # fp32 RNE sums
    slots = np.arange(n * n)
    order = np.lexsort((slots, -keys.astype(np.float64)))
    sel = order[:budget]
    kk = keys[sel].astype(np.float64)
    w = np.exp(kk - kk.max())
    return sel.astype(np.int32), w / w.sum()


@pytest.mark.parametrize("sqrt_n,k,budget,seed", [(8, 4, 4, 0), (8, 8, 8, 1), (16, 6, 5, 2),
                                                   (16, 16, 16, 3), (32, 12, 12, 4), (7, 3, 1, 5)])
def test_addressing_matches_brute_force(sqrt_n, k, budget, seed):
    # with k >= budget and no rounding ties, the product-key result equals the
    # global top-budget over every slot (a pair outside a half's top-k is
    # dominated by >= k >= budget pairs)
    rng = np.random.default_rng(seed)
    P = 64
    s1 = rng.standard_normal((P, sqrt_n)).astype(np.float32)
    s2 = rng.standard_normal((P, sqrt_n)).astype(np.float32)
    idx, wt = oracle.sdm_address(s1, s2, k, budget)
    for p in range(P):
        bi, bw = _brute_top(s1[p], s2[p], budget)
        np.testing.assert_array_equal(idx[p], bi)
        np.testing.assert_allclose(wt[p], bw, rtol=1e-12, atol=0)


def test_addressing_budget_above_k_uses_candidate_set_only():
    # with budget > k the result must come from the k x k candidate grid:
    # brute force restricted to that grid
    rng = np.random.default_rng(7)
    sqrt_n, k, budget = 16, 4, 10
    s1 = rng.standard_normal((32, sqrt_n)).astype(np.float32)
    s2 = rng.standard_normal((32, sqrt_n)).astype(np.float32)
    idx, _ = oracle.sdm_address(s1, s2, k, budget)
    for p in range(32):
        a = np.lexsort((np.arange(sqrt_n), -s1[p].astype(np.float64)))[:k]
        b = np.lexsort((np.arange(sqrt_n), -s2[p].astype(np.float64)))[:k]
        keys = (s1[p][a][:, None] + s2[p][b][None, :]).astype(np.float32).reshape(-1)
        slots = (a[:, None] * sqrt_n + b[None, :]).reshape(-1)
        order = np.lexsort((slots, -keys.astype(np.float64)))[:budget]
        np.testing.assert_array_equal(idx[p], slots[order])


def test_addressing_weights():
    rng = np.random.default_rng(11)
    s1 = rng.standard_normal((16, 8)).astype(np.float32)
    s2 = rng.standard_normal((16, 8)).astype(np.float32)
    _, w1 = oracle.sdm_address(s1, s2, 4, 1)
    assert np.all(w1 == 1.0)
    _, w = oracle.sdm_address(s1, s2, 4, 7)
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=-1) <= 0)  # rank order => non-increasing weights
    # equal keys -> uniform weights
    z = np.zeros((1, 8), np.float32)
    _, wz = oracle.sdm_address(z, z, 4, 8)
    np.testing.assert_array_equal(wz, np.full((1, 8), 1 / 8))


def test_addressing_rounding_tie_goes_to_lowest_slot():
    # half 1 ranks index 1 (1 + 2^-23) above index 0 (1.0); adding 1024 rounds both
    # sums to 1025 in fp32, so the tie is decided by the lower slot: 0*2+0 = 0.
    s1 = np.array([[1.0, 1.0 + 2.0 ** -23]], np.float32)
    s2 = np.array([[1024.0, -5.0]], np.float32)
    idx1, _ = oracle.sdm_address(s1, s2, 2, 1)
    assert idx1.tolist() == [[0]]
    idx2, w2 = oracle.sdm_address(s1, s2, 2, 2)
    assert idx2.tolist() == [[0, 2]]
    np.testing.assert_array_equal(w2, [[0.5, 0.5]])


def test_addressing_signed_zero_ties():
    # -0 and +0 compare equal: ties resolve to the lowest index at both stages
    s1 = np.array([[-0.0, 0.0, -1.0]], np.float32)
    s2 = np.array([[0.0, -0.0, -1.0]], np.float32)
    idx, _ = oracle.sdm_address(s1, s2, 2, 4)
    assert idx.tolist() == [[0, 1, 3, 4]]


def test_unselected_rows_bitwise_unchanged():
    rng = np.random.default_rng(3)
    B, T, H, sqrt_n, dv, k, W, R = 2, 12, 2, 8, 5, 3, 4, 5
    N = sqrt_n * sqrt_n
    sw = [rng.standard_normal((B, T, H, sqrt_n)).astype(np.float32) for _ in range(4)]
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    alpha = rng.uniform(0.9, 1.0, (B, T, H)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, T, H)).astype(np.float32)
    M0 = rng.standard_normal((B, H, N, dv))
    for mode in (0, 1):
        out = oracle.sdm_forward(*sw, v, alpha, beta, M0, k, k, W, R, residual_mode=mode)
        for b in range(B):
            for h in range(H):
                written = set(out["idx_w"][b, :, h].ravel().tolist())
                untouched = [i for i in range(N) if i not in written]
                assert len(untouched) > 0
                np.testing.assert_array_equal(out["M"][b, h, untouched], M0[b, h, untouched])


def test_dense_limit_equals_gdn():
    # every slot selected, raw weights wt_w = k_t and wt_r = q_t, shared residual:
    # the SDM table is then the GDN state S = W^T (row = slot = key channel).
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 2, 9, 3, 6, 4
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    kk = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    alpha = rng.uniform(0.9, 1.0, (B, T, H)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, T, H)).astype(np.float32)
    S0 = rng.standard_normal((B, H, dk, dv))
    perm = rng.permutation(dk).astype(np.int32)  # slot order inside a token is irrelevant
    idx = np.broadcast_to(perm, (B, T, H, dk)).copy()
    wt_w = np.take_along_axis(kk.astype(np.float64), idx.astype(np.int64), axis=-1)
    wt_r = np.take_along_axis(q.astype(np.float64), idx.astype(np.int64), axis=-1)
    M, y = oracle.sdm_recurrence(idx, wt_w, idx, wt_r, v, alpha, beta, S0, residual_mode=0)
    S, o = oracle.gdn(q, kk, v, alpha, beta, S0=S0, kda=False)
    np.testing.assert_allclose(M, S, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y, o, rtol=0, atol=1e-12)
    # the printed per-slot residual (Eq. 4) does not give the dense limit
    M1, _ = oracle.sdm_recurrence(idx, wt_w, idx, wt_r, v, alpha, beta, S0, residual_mode=1)
    assert np.abs(M1 - S).max() > 1e-3
