"""Pins for the SSE oracle: the printed decay-clock example, the reduction to
plain GLA (checked against the unrolled sum), the shared partition and the
routed partitions together against closed-form unrolled sums, the masking
execution as a second algorithm, and the routing invariants."""
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


def _sse_unrolled(logits, q, k, v, lam, topk, q_sh, k_sh, S0):
    """SSE written out as closed-form sums, independent of the oracle's recursion.

    For each (b, h) and partition i let V_i be the tokens that visit it (those
    whose top-k of the logits holds i; every token for the shared partition N)
    and w_t^i the write/read weight (the softmax gate e_t^i for a routed
    partition, 1 for the shared one).  With the visit-restricted cumulative
    log-decay L_i(t) = sum over s in V_i, s <= t of log Lambda_s (one value per
    state row), the state after token t is
        S^i_t = exp(L_i(t)) * S0^i + sum_{j in V_i, j <= t} exp(L_i(t) - L_i(j)) * (w_j^i k_j) v_j^T
    (rows scaled), and o_t = sum_{i in T_t} e_t^i q_t S^i_t + q_sh_t S^N_t.
    Sparse State Expansion slides, "One gate controls both writes and reads"
    (Eqs. 9-14) and "A memory decays only when its partition is visited"; the
    shared partition's weight 1, decay Lambda_t and own q/k are the reading
    under test.
    """
    f64 = lambda a: np.asarray(a, np.float64)
    logits32 = np.asarray(logits, np.float32)
    q, k, v, lam, q_sh, k_sh = map(f64, (q, k, v, lam, q_sh, k_sh))
    B, T, H, N = logits32.shape
    c, d = q.shape[-1], v.shape[-1]
    S = np.array(S0, np.float64, copy=True)
    o = np.zeros((B, T, H, d))
    g = logits32.astype(np.float64)
    e = np.exp(g - g.max(-1, keepdims=True))
    e /= e.sum(-1, keepdims=True)
    # stable sort on the negated fp32 logits: ties keep the lower index first
    sel = np.argsort(-logits32, axis=-1, kind="stable")[..., :topk]
    loglam = np.log(lam)
    for b in range(B):
        for h in range(H):
            for i in range(N + 1):
                if i < N:
                    visits = [t for t in range(T) if i in sel[b, t, h]]
                    w = {t: e[b, t, h, i] for t in visits}
                    keys = k[b, :, h]
                else:
                    visits = list(range(T))
                    w = {t: 1.0 for t in visits}
                    keys = k_sh[b, :, h]
                L = np.zeros((T, c))  # L_i(t), constant between visits
                acc = np.zeros(c)
                for t in range(T):
                    if t in w:
                        acc = acc + loglam[b, t, h]
                    L[t] = acc
                for t in visits:
                    St = np.exp(L[t])[:, None] * S0[b, h, i]
                    for j in visits:
                        if j > t:
                            break
                        St += (np.exp(L[t] - L[j]) * w[j] * keys[j])[:, None] * v[b, j, h][None, :]
                    if i < N:
                        o[b, t, h] += e[b, t, h, i] * (q[b, t, h] @ St)
                    else:
                        o[b, t, h] += q_sh[b, t, h] @ St
                    if t == visits[-1]:
                        S[b, h, i] = St
    return S, o, sel


def test_shared_partition_unrolled_sum():
    # Routed queries zeroed: o is the shared partition's read alone.  The shared
    # partition gets its own key and query (k_sh != k, q_sh != q), a nonzero
    # initial state, and must decay by Lambda_t and take weight 1 on every token.
    B, T, H, N, c, d = 1, 19, 2, 4, 5, 3
    logits, q, k, v, lam = _rand(11, B, T, H, N, c, d)
    rng = np.random.default_rng(12)
    q_sh = rng.standard_normal((B, T, H, c)).astype(np.float32)
    kl = rng.standard_normal((B, T, H, c))
    k_sh = (np.exp(kl) / np.exp(kl).sum(-1, keepdims=True)).astype(np.float32)
    lam = rng.uniform(0.5, 1.0, (B, T, H, c)).astype(np.float32)  # strong decay: visible
    S0 = rng.standard_normal((B, H, N + 1, c, d))
    zq = np.zeros_like(q)
    out = oracle.sse(logits, zq, k, v, lam, topk=2, q_sh=q_sh, k_sh=k_sh, S0=S0)
    S_ref, o_ref, _ = _sse_unrolled(logits, zq, k, v, lam, 2, q_sh, k_sh, S0)
    scale = np.abs(o_ref).max()
    np.testing.assert_allclose(out["o"], o_ref, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(out["S"][:, :, N], S_ref[:, :, N], rtol=0,
                               atol=1e-12 * np.abs(S_ref[:, :, N]).max())
    # the shared read alone: q_sh_t . S^N_t, with S^N_t from the closed form
    assert np.abs(o_ref).max() > 0.1


def test_routed_and_shared_together_unrolled_sum():
    # Both contributions nonzero, several routed partitions with top-2 routing,
    # a separate shared key/query, nonzero initial states in every partition.
    B, T, H, N, c, d = 2, 23, 2, 5, 4, 3
    logits, q, k, v, lam = _rand(13, B, T, H, N, c, d)
    rng = np.random.default_rng(14)
    q_sh = rng.standard_normal((B, T, H, c)).astype(np.float32)
    k_sh = rng.uniform(0.0, 1.0, (B, T, H, c)).astype(np.float32)
    lam = rng.uniform(0.6, 1.0, (B, T, H, c)).astype(np.float32)
    S0 = rng.standard_normal((B, H, N + 1, c, d))
    out = oracle.sse(logits, q, k, v, lam, topk=2, q_sh=q_sh, k_sh=k_sh, S0=S0)
    S_ref, o_ref, sel = _sse_unrolled(logits, q, k, v, lam, 2, q_sh, k_sh, S0)
    np.testing.assert_array_equal(out["sel"], sel)
    np.testing.assert_allclose(out["o"], o_ref, rtol=0, atol=1e-12 * np.abs(o_ref).max())
    np.testing.assert_allclose(out["S"], S_ref, rtol=0, atol=1e-12 * np.abs(S_ref).max())
    # and with the shared projections left out (q_sh = q, k_sh = k by default)
    out2 = oracle.sse(logits, q, k, v, lam, topk=2, S0=S0)
    S_ref2, o_ref2, _ = _sse_unrolled(logits, q, k, v, lam, 2, q, k, S0)
    np.testing.assert_allclose(out2["o"], o_ref2, rtol=0, atol=1e-12 * np.abs(o_ref2).max())
    np.testing.assert_allclose(out2["S"], S_ref2, rtol=0, atol=1e-12 * np.abs(S_ref2).max())
