"""GPU parity of the SSE routing + varlen GLA kernel against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from sparse_state_linear_product_amd import workloads as wl
from tests.helpers import TOL_BF16, TOL_FP32, announce, maxrel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(x, N, topk, S0=None, q_sh=None, k_sh=None, masking=False):
    import sparse_state_linear_product_amd as sslp
    xd = {k: v.to(DEV) for k, v in x.items()}
    B, T, H, _ = x["logits"].shape
    S = (torch.zeros((B, H, N + 1, 128, 128)) if S0 is None else S0.clone()).to(DEV).contiguous()
    sel = torch.empty((B, T, H, topk), dtype=torch.int32, device=DEV)
    e_sel = torch.empty((B, T, H, topk), dtype=torch.float32, device=DEV)
    o = sslp.sse_forward(xd["logits"], xd["q"], xd["k"], xd["v"], xd["lam"], S, topk,
                         q_sh=None if q_sh is None else q_sh.to(DEV),
                         k_sh=None if k_sh is None else k_sh.to(DEV), sel=sel, e_sel=e_sel,
                         masking=masking)
    torch.cuda.synchronize()
    return dict(o=o.cpu(), S=S.cpu(), sel=sel.cpu().numpy(), e_sel=e_sel.cpu().numpy())


def _ref(x, topk, S0=None, q_sh=None, k_sh=None, masking=False):
    n = {k: wl.to_numpy_f32(v) for k, v in x.items()}
    return oracle.sse(n["logits"], n["q"], n["k"], n["v"], n["lam"], topk,
                      q_sh=None if q_sh is None else wl.to_numpy_f32(q_sh),
                      k_sh=None if k_sh is None else wl.to_numpy_f32(k_sh),
                      S0=None if S0 is None else S0.double().numpy(), masking=masking)


def _check(x, N, topk, tag, S0=None, q_sh=None, k_sh=None, masking=False):
    got = _run(x, N, topk, S0, q_sh, k_sh, masking)
    ref = _ref(x, topk, S0, q_sh, k_sh, masking)
    np.testing.assert_array_equal(got["sel"], ref["sel"], err_msg=f"{tag}: selection")
    e_e = np.abs(got["e_sel"] - ref["e_sel"]).max()
    e_o = maxrel(got["o"].double().numpy(), ref["o"], name="o")
    e_S = maxrel(got["S"].double().numpy(), ref["S"], name="S")
    print(f"  {tag}: e_sel {e_e:.2e} o {e_o:.2e} S {e_S:.2e}", flush=True)
    assert e_e <= TOL_FP32
    assert e_o <= TOL_BF16 and e_S <= TOL_BF16, f"{tag}: o {e_o} S {e_S}"
    # partitions never selected by any token keep their state bitwise
    S0n = np.zeros(got["S"].shape, np.float32) if S0 is None else S0.numpy()
    B, T, H, _ = x["logits"].shape
    for b in range(B):
        for h in range(H):
            used = set(ref["sel"][b, :, h].ravel().tolist())
            for i in range(N):
                if i not in used:
                    assert np.array_equal(got["S"].numpy()[b, h, i], S0n[b, h, i])


@pytest.mark.parametrize("T", [1, 23, 64, 130, 400])
def test_sse_small(T):
    announce(f"sse_forward N=8 k=2 B=2 H=2 T={T}")
    x = wl.sse_inputs(wl.SSE, T=T, B=2, H=2, seed=200 + T)
    _check(x, 8, 2, f"sse T={T}")


@pytest.mark.parametrize("N,topk", [(1, 1), (4, 1), (5, 3), (8, 4), (2, 2)])
def test_sse_partition_counts(N, topk):
    announce(f"sse_forward N={N} k={topk}")
    cfg = wl.SseConfig("p", 1, 150, 2, N, topk, 128, 128, torch.bfloat16, 300 + 10 * N + topk)
    x = wl.sse_inputs(cfg)
    _check(x, N, topk, f"N={N} k={topk}")


def test_sse_initial_state_and_separate_shared_qk():
    announce("sse_forward with S0 and separate shared q/k")
    x = wl.sse_inputs(wl.SSE, T=200, B=1, H=2, seed=9)
    g = torch.Generator().manual_seed(10)
    S0 = torch.randn((1, 2, 9, 128, 128), generator=g) * 0.1
    q_sh = torch.randn((1, 200, 2, 128), generator=g).bfloat16()
    k_sh = torch.softmax(torch.randn((1, 200, 2, 128), generator=g), -1).bfloat16()
    _check(x, 8, 2, "S0 + shared q/k", S0=S0, q_sh=q_sh, k_sh=k_sh)


def test_sse_idle_partition_and_unit_decay():
    # one partition is never selected (its state must stay bitwise), and a
    # decay of exactly 1 on a channel with no write keeps that row exactly
    announce("sse idle partition / unit decay channel")
    x = wl.sse_inputs(wl.SSE, T=128, B=1, H=1, seed=12)
    x["logits"][..., 5] = -30.0
    x["lam"][..., 7] = 1.0
    x["k"][..., 7] = 0.0
    g = torch.Generator().manual_seed(13)
    S0 = torch.randn((1, 1, 9, 128, 128), generator=g)
    got = _run(x, 8, 2, S0=S0)
    assert torch.equal(got["S"][0, 0, 5], S0[0, 0, 5])
    assert torch.equal(got["S"][0, 0, :, 7], S0[0, 0, :, 7])


@pytest.mark.parametrize("lo,hi", [(1e-4, 0.05), (0.5, 1.0)])
def test_sse_small_decays(lo, hi):
    # decays anywhere in (0, 1]: with U(1e-4, 0.05) a block's product of decays
    # leaves the fp32 range after a few visits, so blocks are cut short; the
    # result must still match the oracle (grouped and masked executions)
    announce(f"sse_forward with Lambda ~ U({lo}, {hi})")
    x = wl.sse_inputs(wl.SSE, T=150, B=1, H=2, seed=int(40 + 1e4 * lo))
    g = torch.Generator().manual_seed(41)
    x["lam"] = torch.empty(x["lam"].shape).uniform_(lo, hi, generator=g)
    S0 = torch.randn((1, 2, 9, 128, 128), generator=g) * 0.1
    _check(x, 8, 2, f"Lambda U({lo},{hi})", S0=S0)
    _check(x, 8, 2, f"masking, Lambda U({lo},{hi})", S0=S0, masking=True)


@pytest.mark.slow
def test_sse_full_config():
    cfg = wl.SSE
    announce(f"{cfg.name} full size")
    x = wl.sse_inputs(cfg)
    _check(x, cfg.N, cfg.topk, cfg.name)


# ---------------- masking execution ----------------

@pytest.mark.parametrize("N,topk,T", [(8, 2, 1), (8, 2, 23), (8, 2, 130), (5, 3, 70), (4, 1, 65),
                                      (8, 4, 64)])
def test_sse_masking_matches_masking_oracle(N, topk, T):
    announce(f"sse_forward_masking N={N} k={topk} T={T}")
    cfg = wl.SseConfig("m", 2, T, 2, N, topk, 128, 128, torch.bfloat16, 900 + 10 * N + topk + T)
    x = wl.sse_inputs(cfg)
    _check(x, N, topk, f"masking N={N} k={topk} T={T}", masking=True)


def test_sse_masking_agrees_with_varlen_and_keeps_idle_states():
    # the two executions compute the same thing: identical routing, outputs
    # and states within the bf16 bound, and a never-selected partition (all of
    # its steps masked, decay frozen at 1) keeps its state bitwise
    announce("sse_forward_masking vs sse_forward, S0 and separate shared q/k")
    x = wl.sse_inputs(wl.SSE, T=200, B=1, H=2, seed=31)
    x["logits"][..., 6] = -30.0
    g = torch.Generator().manual_seed(32)
    S0 = torch.randn((1, 2, 9, 128, 128), generator=g) * 0.1
    q_sh = torch.randn((1, 200, 2, 128), generator=g).bfloat16()
    k_sh = torch.softmax(torch.randn((1, 200, 2, 128), generator=g), -1).bfloat16()
    a = _run(x, 8, 2, S0, q_sh, k_sh, masking=True)
    b = _run(x, 8, 2, S0, q_sh, k_sh, masking=False)
    np.testing.assert_array_equal(a["sel"], b["sel"])
    np.testing.assert_array_equal(a["e_sel"], b["e_sel"])
    e_o = maxrel(a["o"].double().numpy(), b["o"].double().numpy(), name="o")
    e_S = maxrel(a["S"].double().numpy(), b["S"].double().numpy(), name="S")
    print(f"  masking vs varlen: o {e_o:.2e} S {e_S:.2e}", flush=True)
    assert e_o <= TOL_BF16 and e_S <= TOL_BF16
    assert torch.equal(a["S"][0, :, 6], S0[0, :, 6])
    # the shared partition runs the same steps in both executions
    assert torch.equal(a["S"][0, :, 8], b["S"][0, :, 8])
    ref = _ref(x, 2, S0, q_sh, k_sh, masking=True)
    assert maxrel(a["o"].double().numpy(), ref["o"], name="o") <= TOL_BF16


# ---------------- decode step (one token per sequence) ----------------

def _decode_run(x, N, topk, S0, q_sh=None, k_sh=None):
    import sparse_state_linear_product_amd as sslp
    B, T, H, _ = x["logits"].shape
    S = S0.clone().to(DEV).contiguous()
    os, sels, es = [], [], []
    for t in range(T):
        st = {k: v[:, t].contiguous().to(DEV) for k, v in x.items()}
        sel = torch.empty((B, H, topk), dtype=torch.int32, device=DEV)
        e_sel = torch.empty((B, H, topk), dtype=torch.float32, device=DEV)
        o = sslp.sse_decode_step(st["logits"], st["q"], st["k"], st["v"], st["lam"], S, topk,
                                 q_sh=None if q_sh is None else q_sh[:, t].contiguous().to(DEV),
                                 k_sh=None if k_sh is None else k_sh[:, t].contiguous().to(DEV),
                                 sel=sel, e_sel=e_sel)
        os.append(o)
        sels.append(sel)
        es.append(e_sel)
    torch.cuda.synchronize()
    return dict(o=torch.stack(os, 1).cpu(), S=S.cpu(), sel=torch.stack(sels, 1).cpu().numpy(),
                e_sel=torch.stack(es, 1).cpu().numpy())


@pytest.mark.parametrize("N,topk,B,H,T", [(8, 2, 3, 2, 6), (5, 3, 2, 3, 4), (1, 1, 2, 1, 3),
                                          (8, 4, 1, 2, 5)])
def test_sse_decode_steps_match_oracle(N, topk, B, H, T):
    announce(f"sse_decode_step N={N} k={topk} B={B} H={H} steps={T}")
    cfg = wl.SseConfig("dec", B, T, H, N, topk, 128, 128, torch.bfloat16, 700 + 10 * N + topk)
    x = wl.sse_inputs(cfg)
    g = torch.Generator().manual_seed(701 + N)
    S0 = torch.randn((B, H, N + 1, 128, 128), generator=g) * 0.1
    got = _decode_run(x, N, topk, S0)
    ref = _ref(x, topk, S0)
    np.testing.assert_array_equal(got["sel"], ref["sel"], err_msg="decode selection")
    e_e = np.abs(got["e_sel"] - ref["e_sel"]).max()
    e_o = maxrel(got["o"].double().numpy(), ref["o"], name="o")
    e_S = maxrel(got["S"].double().numpy(), ref["S"], name="S")
    print(f"  decode N={N} k={topk}: e_sel {e_e:.2e} o {e_o:.2e} S {e_S:.2e}", flush=True)
    assert e_e <= TOL_FP32
    assert e_o <= TOL_BF16 and e_S <= TOL_BF16


def test_sse_decode_touches_only_selected_states_and_separate_shared_qk():
    announce("sse_decode_step: untouched states bitwise, separate shared q/k")
    B, H, N, topk = 2, 3, 8, 2
    cfg = wl.SseConfig("dec1", B, 1, H, N, topk, 128, 128, torch.bfloat16, 777)
    x = wl.sse_inputs(cfg)
    g = torch.Generator().manual_seed(778)
    S0 = torch.randn((B, H, N + 1, 128, 128), generator=g)
    q_sh = torch.randn((B, 1, H, 128), generator=g).bfloat16()
    k_sh = torch.softmax(torch.randn((B, 1, H, 128), generator=g), -1).bfloat16()
    got = _decode_run(x, N, topk, S0, q_sh=q_sh, k_sh=k_sh)
    ref = _ref(x, topk, S0, q_sh=q_sh, k_sh=k_sh)
    np.testing.assert_array_equal(got["sel"], ref["sel"])
    assert maxrel(got["o"].double().numpy(), ref["o"], name="o") <= TOL_BF16
    assert maxrel(got["S"].double().numpy(), ref["S"], name="S") <= TOL_BF16
    for b in range(B):
        for h in range(H):
            used = set(got["sel"][b, 0, h].tolist()) | {N}
            for i in range(N + 1):
                if i not in used:
                    assert torch.equal(got["S"][b, h, i], S0[b, h, i]), (b, h, i)


@pytest.mark.slow
def test_sse_decode_full_size():
    # the decode workload: 64 sequences x 16 heads, 8 routed + 1 shared states of
    # 128 x 128 (seeded background), two steps in the configuration the
    # benchmark times; every state slice, output and selection against the oracle
    cfg = wl.SSE_DECODE
    announce(f"{cfg.name} full size, 2 steps")
    x = wl.sse_inputs(cfg, T=2)
    g = torch.Generator().manual_seed(cfg.seed + 3)
    S0 = torch.randn((cfg.B, cfg.H, cfg.N + 1, cfg.c, cfg.d), generator=g)
    got = _decode_run(x, cfg.N, cfg.topk, S0)
    ref = _ref(x, cfg.topk, S0)
    np.testing.assert_array_equal(got["sel"], ref["sel"])
    e_o = maxrel(got["o"].double().numpy(), ref["o"], name="o")
    e_S = maxrel(got["S"].double().numpy(), ref["S"], name="S")
    print(f"  {cfg.name}: o {e_o:.2e} S {e_S:.2e}", flush=True)
    assert e_o <= TOL_BF16 and e_S <= TOL_BF16
    # partitions selected by neither step are untouched
    for b in range(0, cfg.B, 7):
        for h in range(cfg.H):
            used = set(got["sel"][b, :, h].ravel().tolist()) | {cfg.N}
            for i in range(cfg.N + 1):
                if i not in used:
                    assert torch.equal(got["S"][b, h, i], S0[b, h, i])
