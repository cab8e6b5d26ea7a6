"""Pins for the SSE oracle: the printed decay-clock example, the reduction to
plain GLA (checked against the unrolled sum), the masking execution as a
second algorithm, and the routing invariants."""
import json
import os

import numpy as np

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, B, T, H, N, c, d):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((B, T, H, N)).astype(np.float32)
    q = rng.standard_normal((B, T, H, c)).astype(np.float32)
    kl = rng.standard_normal((B, T, H, c))
    k = (np.exp(kl) / np.exp(kl).sum(-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, T, H, d)).astype(np.float32)
    lam = rng.uniform(0.95, 1.0, (B, T, H, c)).astype(np.float32)
    return logits, q, k, v, lam


def test_decay_clock_example():
    with open(os.path.join(GOLD, "sse_decay_clock.json")) as f:
        g = json.load(f)
    # one write of 1 into partition 0 at t=0, then 100 tokens with v = 0 of which
    # 10 visit partition 0 (the rest visit partition 1): its content decays 10 times
    T = 1 + g["dense_decay_events"]
    visits = set(range(1, T, g["dense_decay_events"] // g["sparse_decay_events"]))
    assert len(visits) == g["sparse_decay_events"]
    logits = np.zeros((1, T, 1, 2), np.float32)
    for t in range(T):
        logits[0, t, 0] = [5.0, 0.0] if (t == 0 or t in visits) else [0.0, 5.0]
    ones = np.ones((1, T, 1, 1), np.float32)
    v = np.zeros((1, T, 1, 1), np.float32)
    v[0, 0] = 1.0
    lam = np.full((1, T, 1, 1), g["decay"], np.float32)
    out = oracle.sse(logits, ones, ones, v, lam, topk=1)
    e0 = out["e_sel"][0, 0, 0, 0]
    retained = out["S"][0, 0, 0, 0, 0] / e0  # the t=0 write itself is not decayed
    assert round(retained, g["printed_digits"]) == g["sparse_retained_printed"]
    # dense reference: a single partition visited by every token
    out_d = oracle.sse(np.zeros((1, T, 1, 1), np.float32), ones, ones, v, lam, topk=1,
                       k_sh=np.zeros_like(ones))
    retained_d = out_d["S"][0, 0, 0, 0, 0]
    assert round(retained_d, g["printed_digits"]) == g["dense_retained_printed"]


def test_single_partition_reduces_to_gla_unrolled_sum():
    # N = 1, k = 1 (gate weight exactly 1) and a zero shared key/query: plain GLA,
    # o_t = sum_{j<=t} sum_r q_t[r] (prod_{s=j+1..t} lam_s[r]) k_j[r] v_j
    B, T, H, c, d = 1, 13, 2, 5, 4
    _, q, k, v, lam = _rand(2, B, T, H, 1, c, d)
    logits = np.zeros((B, T, H, 1), np.float32)
    z = np.zeros_like(q)
    out = oracle.sse(logits, q, k, v, lam, topk=1, q_sh=z, k_sh=z)
    assert np.all(out["e_sel"] == 1.0)
    L = np.log(lam.astype(np.float64))
    for h in range(H):
        for t in range(T):
            acc = np.zeros(d)
            for j in range(t + 1):
                dec = np.exp(L[0, j + 1:t + 1, h].sum(axis=0))  # [c]
                acc += (q[0, t, h] * dec * k[0, j, h]).sum() * v[0, j, h]
            np.testing.assert_allclose(out["o"][0, t, h], acc, rtol=0, atol=1e-12)
    assert np.all(out["S"][:, :, 1] == 0.0)  # shared state never written


def test_masking_execution_matches_definition():
    args = _rand(3, 2, 40, 3, 8, 6, 5)
    S0 = np.random.default_rng(4).standard_normal((2, 3, 9, 6, 5))
    a = oracle.sse(*args, topk=2, S0=S0)
    b = oracle.sse(*args, topk=2, S0=S0, masking=True)
    np.testing.assert_allclose(a["o"], b["o"], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(a["S"], b["S"])


def test_routing_invariants():
    logits, q, k, v, lam = _rand(5, 2, 30, 2, 8, 4, 3)
    logits[..., 6] = -30.0  # partition 6 is never selected
    S0 = np.random.default_rng(6).standard_normal((2, 2, 9, 4, 3))
    out = oracle.sse(logits, q, k, v, lam, topk=2, S0=S0)
    # selected gate mass is at most one and is not renormalised
    mass = out["e_sel"].sum(-1)
    assert np.all(mass <= 1.0 + 1e-15) and np.all(mass < 1.0)
    # selection = top-2 of the softmax, ties to the lowest index
    e = np.exp(logits.astype(np.float64))
    e /= e.sum(-1, keepdims=True)
    for idx in np.ndindex(*logits.shape[:-1]):
        order = np.lexsort((np.arange(8), -e[idx]))[:2]
        assert out["sel"][idx].tolist() == order.tolist()
        np.testing.assert_allclose(out["e_sel"][idx], e[idx][order], rtol=1e-13)
    # an unvisited partition keeps its state bitwise, decay included
    np.testing.assert_array_equal(out["S"][:, :, 6], S0[:, :, 6])


def test_unit_decay_channel_retains_exactly():
    # Proposition 4 (backup slide): a channel with decay exactly 1 and no write
    # keeps its content exactly over any number of visits
    logits, q, k, v, lam = _rand(7, 1, 50, 1, 2, 4, 3)
    lam[..., 2] = 1.0
    k[..., 2] = 0.0
    S0 = np.random.default_rng(8).standard_normal((1, 1, 3, 4, 3))
    out = oracle.sse(logits, q, k, v, lam, topk=1, S0=S0)
    np.testing.assert_array_equal(out["S"][0, 0, :, 2], S0[0, 0, :, 2])
