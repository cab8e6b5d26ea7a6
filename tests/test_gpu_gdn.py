"""GPU parity of the chunked GDN / KDA kernel against the sequential fp64 oracle."""
import numpy as np
import pytest

import oracle
from sparse_state_linear_product_amd import workloads as wl
from tests.helpers import TOL_BF16, announce, maxrel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(x, S0=None, inplace=False):
    import sparse_state_linear_product_amd as sslp
    xd = {k: v.to(DEV) for k, v in x.items()}
    S0d = None if S0 is None else S0.to(DEV).contiguous()
    S_out = S0d if inplace else None
    o, S = sslp.gdn_chunk_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], S0=S0d,
                                  S_out=S_out)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu()


def _ref(x, S0, kda):
    n = {k: wl.to_numpy_f32(v) for k, v in x.items()}
    return oracle.gdn(n["q"], n["k"], n["v"], n["alpha"], n["beta"],
                      S0=None if S0 is None else S0.double().numpy(), kda=kda)


def _check(x, kda, S0=None, inplace=False, tag=""):
    o, S = _run(x, S0, inplace)
    Sr, orf = _ref(x, S0, kda)
    e_o = maxrel(o.double().numpy(), orf, name="o")
    e_S = maxrel(S.double().numpy(), Sr, name="S")
    print(f"  {tag}: o {e_o:.2e} S {e_S:.2e}", flush=True)
    assert np.isfinite(o.float().numpy()).all() and np.isfinite(S.numpy()).all()
    assert e_o <= TOL_BF16 and e_S <= TOL_BF16, f"{tag}: o {e_o} S {e_S}"
    return e_o, e_S


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("T", [1, 17, 64, 100, 300])
def test_gdn_small(kda, T):
    cfg = wl.KDA if kda else wl.GDN
    announce(f"gdn_chunk_forward kda={kda} B=2 H=3 T={T}")
    x = wl.gdn_inputs(cfg, T=T, B=2, H=3, seed=100 + T)
    _check(x, kda, tag=f"{'kda' if kda else 'gdn'} T={T}")


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_gdn_initial_state_in_place(kda):
    cfg = wl.KDA if kda else wl.GDN
    announce(f"gdn_chunk_forward with S0, in place, kda={kda}")
    x = wl.gdn_inputs(cfg, T=150, B=1, H=2, seed=7)
    S0 = torch.randn((1, 2, 128, 128), generator=torch.Generator().manual_seed(3)) * 0.5
    _check(x, kda, S0=S0, inplace=True, tag="S0 in place")


def test_kda_uniform_channels_matches_gdn():
    import sparse_state_linear_product_amd as sslp
    announce("kda(alpha*1) vs gdn on the GPU")
    x = wl.gdn_inputs(wl.GDN, T=200, B=1, H=2, seed=11)
    xd = {k: v.to(DEV) for k, v in x.items()}
    a_ch = xd["alpha"][..., None].expand(-1, -1, -1, 128).contiguous()
    o1, S1 = sslp.gdn_chunk_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"])
    o2, S2 = sslp.gdn_chunk_forward(xd["q"], xd["k"], xd["v"], a_ch, xd["beta"])
    torch.cuda.synchronize()
    assert maxrel(o2.cpu().double().numpy(), o1.cpu().double().numpy(), name="o2") <= 1e-2
    assert maxrel(S2.cpu().double().numpy(), S1.cpu().double().numpy(), name="S2") <= 1e-2


def test_gdn_empty_sequence_copies_state():
    import sparse_state_linear_product_amd as sslp
    x = wl.gdn_inputs(wl.GDN, T=0, B=1, H=1, seed=1)
    S0 = torch.randn((1, 1, 128, 128), device=DEV)
    xd = {k: v.to(DEV) for k, v in x.items()}
    _, S = sslp.gdn_chunk_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], S0=S0)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)


@pytest.mark.slow
@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_gdn_full_config(kda):
    cfg = wl.KDA if kda else wl.GDN
    announce(f"{cfg.name} full size")
    x = wl.gdn_inputs(cfg)
    _check(x, kda, tag=cfg.name)


# ---------------- GDN2: erase vector b, write vector w ----------------

def _run2(x, S0=None):
    import sparse_state_linear_product_amd as sslp
    xd = {k: v.to(DEV) for k, v in x.items()}
    o, S = sslp.gdn2_chunk_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["erase"],
                                   xd["write"], S0=None if S0 is None else S0.to(DEV).contiguous())
    torch.cuda.synchronize()
    return o.cpu(), S.cpu()


def _ref2(x, S0=None):
    n = {k: wl.to_numpy_f32(v) for k, v in x.items()}
    return oracle.gdn2(n["q"], n["k"], n["v"], n["alpha"], n["erase"], n["write"],
                       S0=None if S0 is None else S0.double().numpy())


@pytest.mark.parametrize("T", [1, 17, 64, 100, 300])
def test_gdn2_small(T):
    announce(f"gdn2_chunk_forward B=2 H=3 T={T}")
    x = wl.gdn2_inputs(wl.GDN2, T=T, B=2, H=3, seed=500 + T)
    o, S = _run2(x)
    Sr, orf = _ref2(x)
    e_o, e_S = maxrel(o.double().numpy(), orf, name="o"), maxrel(S.double().numpy(), Sr, name="S")
    print(f"  gdn2 T={T}: o {e_o:.2e} S {e_S:.2e}", flush=True)
    assert np.isfinite(o.float().numpy()).all() and np.isfinite(S.numpy()).all()
    assert e_o <= TOL_BF16 and e_S <= TOL_BF16


@pytest.mark.parametrize("mode", ["gdn", "kda", "gdn2"])
@pytest.mark.parametrize("B,H,T", [(1, 3, 129), (3, 1, 260), (1, 1, 64 * 7 + 5)])
def test_gdn_head_counts_off_the_xcd_grouping(mode, B, H, T):
    # an odd number of (batch, head) pairs gives a state grid that is not a
    # multiple of the 8 XCDs (workgroups keep their launch order), and 3 to 8
    # chunks exercise the record pulled into L2 two chunks ahead near the end
    announce(f"{mode} B={B} H={H} T={T}")
    if mode == "gdn2":
        x = wl.gdn2_inputs(wl.GDN2, T=T, B=B, H=H, seed=700 + T)
        o, S = _run2(x)
        Sr, orf = _ref2(x)
        e_o, e_S = maxrel(o.double().numpy(), orf, name="o"), maxrel(S.double().numpy(), Sr, name="S")
        assert np.isfinite(o.float().numpy()).all() and np.isfinite(S.numpy()).all()
        assert e_o <= TOL_BF16 and e_S <= TOL_BF16, f"o {e_o} S {e_S}"
    else:
        kda = mode == "kda"
        x = wl.gdn_inputs(wl.KDA if kda else wl.GDN, T=T, B=B, H=H, seed=600 + T)
        _check(x, kda, tag=f"{mode} B={B} H={H} T={T}")


def test_gdn2_with_initial_state_and_kda_reduction():
    # with S0; and b = w = beta on every channel, which the slide states is KDA
    announce("gdn2_chunk_forward with S0; b = w = beta 1 vs the KDA oracle")
    x = wl.gdn2_inputs(wl.GDN2, T=150, B=1, H=2, seed=41)
    S0 = torch.randn((1, 2, 128, 128), generator=torch.Generator().manual_seed(42)) * 0.5
    o, S = _run2(x, S0)
    Sr, orf = _ref2(x, S0)
    assert maxrel(o.double().numpy(), orf, name="o") <= TOL_BF16
    assert maxrel(S.double().numpy(), Sr, name="S") <= TOL_BF16
    x["erase"] = x["beta"][..., None].expand(-1, -1, -1, 128).contiguous()
    x["write"] = x["beta"][..., None].expand(-1, -1, -1, 128).contiguous()
    o, S = _run2(x, S0)
    n = {k: wl.to_numpy_f32(v) for k, v in x.items()}
    Sk, ok = oracle.gdn(n["q"], n["k"], n["v"], n["alpha"], n["beta"], S0=S0.double().numpy(),
                        kda=True)
    e_o, e_S = maxrel(o.double().numpy(), ok, name="o"), maxrel(S.double().numpy(), Sk, name="S")
    print(f"  gdn2 as KDA: o {e_o:.2e} S {e_S:.2e}", flush=True)
    assert e_o <= TOL_BF16 and e_S <= TOL_BF16


def test_gdn2_empty_sequence_copies_state():
    import sparse_state_linear_product_amd as sslp
    announce("gdn2_chunk_forward T=0")
    x = wl.gdn2_inputs(wl.GDN2, T=0, B=1, H=2, seed=43)
    S0 = torch.randn((1, 2, 128, 128), generator=torch.Generator().manual_seed(44))
    xd = {k: v.to(DEV) for k, v in x.items()}
    o, S = sslp.gdn2_chunk_forward(xd["q"], xd["k"], xd["v"], xd["alpha"], xd["erase"], xd["write"],
                                   S0=S0.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), S0)


@pytest.mark.slow
def test_gdn2_full_config():
    # B=4, T=4096, H=16, d=128 against the sequential fp64 oracle
    cfg = wl.GDN2
    announce(f"{cfg.name} full size")
    x = wl.gdn2_inputs(cfg)
    o, S = _run2(x)
    Sr, orf = _ref2(x)
    e_o = maxrel(o.double().numpy(), orf, name="o")
    e_S = maxrel(S.double().numpy(), Sr, name="S")
    print(f"  {cfg.name}: o {e_o:.2e} S {e_S:.2e}", flush=True)
    assert e_o <= TOL_BF16 and e_S <= TOL_BF16


@pytest.mark.parametrize("mode", ["gdn", "kda", "gdn2"])
def test_strong_decays_at_the_documented_bound(mode):
    # decays drawn from U(2^-4, 0.2) (per token for GDN, per channel for KDA and
    # GDN2): products of decays within a 16-token block reach 2^-60, the edge of
    # the range the chunked factorisation is exact for; parity must hold
    announce(f"{mode} with decays ~ U(1/16, 0.2)")
    g = torch.Generator().manual_seed(77)
    S0 = torch.randn((1, 2, 128, 128), generator=g) * 0.5
    if mode == "gdn2":
        x = wl.gdn2_inputs(wl.GDN2, T=130, B=1, H=2, seed=78)
        x["alpha"] = torch.empty(x["alpha"].shape).uniform_(1.0 / 16, 0.2, generator=g)
        o, S = _run2(x, S0)
        Sr, orf = _ref2(x, S0)
        e_o, e_S = maxrel(o.double().numpy(), orf, name="o"), maxrel(S.double().numpy(), Sr, name="S")
        assert np.isfinite(o.float().numpy()).all() and np.isfinite(S.numpy()).all()
        assert e_o <= TOL_BF16 and e_S <= TOL_BF16, f"gdn2: o {e_o} S {e_S}"
    else:
        kda = mode == "kda"
        x = wl.gdn_inputs(wl.KDA if kda else wl.GDN, T=130, B=1, H=2, seed=79)
        x["alpha"] = torch.empty(x["alpha"].shape).uniform_(1.0 / 16, 0.2, generator=g)
        _check(x, kda, S0=S0, tag=f"{mode} strong decay")


@pytest.mark.parametrize("mode", ["gdn", "kda", "gdn2"])
def test_tiny_decays_stay_finite(mode):
    # below the documented bound (per-channel decays down to 1e-4) the chunked
    # form must not produce inf or NaN; the scalar decay (GDN) stays exact there
    announce(f"{mode} with decays ~ U(1e-4, 0.05)")
    g = torch.Generator().manual_seed(80)
    if mode == "gdn2":
        x = wl.gdn2_inputs(wl.GDN2, T=100, B=1, H=2, seed=81)
        x["alpha"] = torch.empty(x["alpha"].shape).uniform_(1e-4, 0.05, generator=g)
        o, S = _run2(x)
    else:
        x = wl.gdn_inputs(wl.KDA if mode == "kda" else wl.GDN, T=100, B=1, H=2, seed=82)
        x["alpha"] = torch.empty(x["alpha"].shape).uniform_(1e-4, 0.05, generator=g)
        if mode == "gdn":
            _check(x, False, tag="gdn tiny decay")
            return
        o, S = _run(x)
    assert np.isfinite(o.float().numpy()).all() and np.isfinite(S.numpy()).all()
