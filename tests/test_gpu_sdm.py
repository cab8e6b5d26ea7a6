"""GPU parity of the Sparse Delta Memory path (addressing, update/read, decode)
against the fp64 oracle, through the C ABI."""
import dataclasses

import numpy as np
import pytest

import oracle
from sparse_state_linear_product_amd import workloads as wl
from tests.helpers import TOL_BF16, TOL_FP32, announce, maxrel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _sslp():
    import sparse_state_linear_product_amd as sslp
    return sslp


def _np(t):
    return wl.to_numpy_f32(t)


def _run_forward(cfg, x, M0, mode, T=None):
    sslp = _sslp()
    T = x["sw1"].shape[1]
    xd = {k: v.to(DEV) for k, v in x.items()}
    M = M0.to(DEV).float().contiguous()
    shp = (cfg.B, T, cfg.H)
    idx_w = torch.empty(shp + (cfg.W,), dtype=torch.int32, device=DEV)
    wt_w = torch.empty(shp + (cfg.W,), dtype=torch.float32, device=DEV)
    idx_r = torch.empty(shp + (cfg.R,), dtype=torch.int32, device=DEV)
    wt_r = torch.empty(shp + (cfg.R,), dtype=torch.float32, device=DEV)
    y = sslp.sdm_forward(xd["sw1"], xd["sw2"], xd["sr1"], xd["sr2"], xd["v"], xd["alpha"],
                         xd["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R, residual_mode=mode,
                         idx_w=idx_w, wt_w=wt_w, idx_r=idx_r, wt_r=wt_r)
    torch.cuda.synchronize()
    return dict(y=y.cpu(), M=M.cpu(), idx_w=idx_w.cpu().numpy(), wt_w=wt_w.cpu().numpy(),
                idx_r=idx_r.cpu().numpy(), wt_r=wt_r.cpu().numpy())


def _oracle_forward(cfg, x, M0, mode):
    n = {k: _np(v) for k, v in x.items()}
    return oracle.sdm_forward(n["sw1"], n["sw2"], n["sr1"], n["sr2"], n["v"], n["alpha"],
                              n["beta"], M0.double().numpy(), cfg.k_w, cfg.k_r, cfg.W, cfg.R,
                              residual_mode=mode)


def _check(cfg, got, ref, M0, tag):
    np.testing.assert_array_equal(got["idx_w"], ref["idx_w"], err_msg=f"{tag}: write indices")
    np.testing.assert_array_equal(got["idx_r"], ref["idx_r"], err_msg=f"{tag}: read indices")
    e_w = np.abs(got["wt_w"] - ref["wt_w"]).max()
    e_r = np.abs(got["wt_r"] - ref["wt_r"]).max()
    e_y = maxrel(got["y"].double().numpy(), ref["y"], name="y")
    e_M = maxrel(got["M"].double().numpy(), ref["M"], name="M")
    print(f"  {tag}: wt_w {e_w:.2e} wt_r {e_r:.2e} y {e_y:.2e} M {e_M:.2e}", flush=True)
    assert e_w <= TOL_FP32 and e_r <= TOL_FP32
    # the table arithmetic is fp32 whatever the input dtype; y is rounded to the io dtype
    assert e_M <= TOL_FP32, f"{tag}: M error {e_M}"
    assert e_y <= (TOL_FP32 if cfg.dtype == torch.float32 else TOL_BF16), f"{tag}: y error {e_y}"
    # rows outside every write set are bitwise untouched
    Mg, M0n = got["M"].numpy(), M0.float().numpy()
    for b in range(cfg.B):
        for h in range(cfg.H):
            written = np.zeros(cfg.N, bool)
            written[np.unique(ref["idx_w"][b, :, h])] = True
            assert np.array_equal(Mg[b, h, ~written], M0n[b, h, ~written]), f"{tag}: untouched rows"


@pytest.mark.parametrize("mode", [0, 1])
def test_sdm_tiny_config(mode):
    cfg = wl.SDM_TINY
    announce(f"sdm tiny fp32 T={cfg.T} mode={mode}")
    x = wl.sdm_inputs(cfg)
    M0 = torch.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v))
    got = _run_forward(cfg, x, M0, mode)
    ref = _oracle_forward(cfg, x, M0, mode)
    _check(cfg, got, ref, M0, f"tiny mode {mode}")


SMALL = [
    # B, T, H, sqrtN, d_v, k_w, k_r, W, R, dtype, mode
    (2, 50, 3, 16, 20, 6, 5, 7, 9, "f32", 0),
    (1, 33, 2, 13, 36, 13, 3, 64, 9, "f32", 1),
    (1, 40, 1, 100, 64, 32, 8, 32, 40, "bf16", 0),
    (1, 24, 2, 240, 32, 32, 32, 32, 32, "bf16", 0),
    (1, 6, 1, 1000, 8, 64, 64, 128, 128, "f32", 0),
    (3, 17, 1, 5, 4, 5, 2, 25, 1, "f32", 0),
    (1, 1, 1, 1, 4, 1, 1, 1, 1, "f32", 0),
    # W = R = 32 and T >= 64 take the pipelined kernel: ragged token blocks,
    # tiny tables (every token's rows collide with the last few tokens' writes,
    # so nearly every row is forwarded), several column slices
    (2, 100, 2, 8, 24, 8, 8, 32, 32, "f32", 0),
    (1, 65, 1, 6, 16, 6, 6, 32, 32, "bf16", 1),
    (1, 64, 2, 7, 8, 7, 7, 32, 32, "f32", 1),
    (1, 300, 3, 240, 40, 32, 32, 32, 32, "bf16", 0),
    (1, 177, 1, 40, 32, 16, 16, 32, 32, "bf16", 1),
    # mid-size tables: tens of forwarded rows per chunk, and around the in-LDS
    # forward capacity (some chunks pass rows through LDS, others patch directly)
    (1, 200, 2, 100, 16, 32, 32, 32, 32, "f32", 0),
    (1, 160, 1, 64, 24, 32, 32, 32, 32, "bf16", 1),
    # more column slices (B*H*d_v/8 = 1200) than the chip holds workgroups at
    # once: the slices run in several rounds
    (5, 80, 2, 64, 960, 32, 32, 32, 32, "bf16", 0),
    # W = R = 64 and T >= 64: the pipelined kernel in chunks of 8 tokens (a
    # 64-bit mask per token, one column per compute lane): tiny tables where
    # nearly every row is forwarded, ragged tails, mid-size and 1.4B-size tables
    (2, 100, 2, 10, 24, 10, 10, 64, 64, "f32", 0),
    (1, 67, 1, 9, 16, 9, 9, 64, 64, "bf16", 1),
    (1, 64, 2, 12, 8, 12, 12, 64, 64, "f32", 1),
    (1, 200, 2, 100, 16, 64, 64, 64, 64, "f32", 0),
    (1, 161, 1, 64, 24, 64, 64, 64, 64, "bf16", 1),
    (1, 300, 3, 240, 40, 64, 64, 64, 64, "bf16", 0),
    (2, 72, 2, 64, 960, 64, 64, 64, 64, "bf16", 0),
]


@pytest.mark.parametrize("case", SMALL)
def test_sdm_small_shapes(case):
    B, T, H, sq, dv, kw, kr, W, R, dt, mode = case
    dtype = torch.float32 if dt == "f32" else torch.bfloat16
    cfg = wl.SdmConfig("small", B, T, H, sq, dv, kw, kr, W, R, dtype, 77 + sum(case[:9]))
    announce(f"sdm small {case}")
    x = wl.sdm_inputs(cfg)
    M0 = torch.randn((B, H, sq * sq, dv), generator=torch.Generator().manual_seed(5))
    got = _run_forward(cfg, x, M0, mode)
    ref = _oracle_forward(cfg, x, M0, mode)
    _check(cfg, got, ref, M0, f"small {case}")


def _address_cases():
    r = np.random.default_rng(123)
    cases = []
    # rounding tie: fp32 sums 1+2^-23+1024 and 1+1024 both round to 1025
    s1 = np.array([1.0, 1.0 + 2.0 ** -23], np.float32)
    s2 = np.array([1024.0, -5.0], np.float32)
    cases.append(("rounding_tie", s1[None, None, None], s2[None, None, None], 2, 1))
    cases.append(("rounding_tie_2", s1[None, None, None], s2[None, None, None], 2, 2))
    cases.append(("signed_zero", np.array([[[[-0.0, 0.0, -1.0]]]], np.float32),
                  np.array([[[[0.0, -0.0, -1.0]]]], np.float32), 2, 4))
    # heavy ties: scores from a 7-value set
    q1 = r.integers(-3, 4, (4, 64, 2, 240)).astype(np.float32)
    q2 = r.integers(-3, 4, (4, 64, 2, 240)).astype(np.float32)
    cases.append(("quantized_240_k32_w32", q1, q2, 32, 32))
    cases.append(("quantized_240_k16_w100", q1, q2, 16, 100))
    z = np.zeros((1, 3, 1, 50), np.float32)
    cases.append(("all_equal", z, z, 10, 37))
    g1 = r.standard_normal((2, 100, 2, 240)).astype(np.float32)
    g2 = r.standard_normal((2, 100, 2, 240)).astype(np.float32)
    cases.append(("gauss_240_k32_w32", g1, g2, 32, 32))
    cases.append(("gauss_240_k8_w64", g1, g2, 8, 64))
    # one workgroup per problem with k > 32 (one candidate row per lane pass) and
    # dominance sets of more than 128 entries (merged from four sorted lists)
    cases.append(("gauss_240_k40_w40_D158", g1, g2, 40, 40))
    cases.append(("quantized_240_k48_w64_D248", q1, q2, 48, 64))
    cases.append(("quantized_240_k64_w48_D198", q1, q2, 64, 48))
    cases.append(("gauss_240_k33_w33_D123", g1, g2, 33, 33))
    # more than 1024 problems: the one-wavefront-per-problem kernel (fewer: one
    # workgroup per problem); the same exact selection either way
    q3 = r.integers(-3, 4, (2, 400, 2, 240)).astype(np.float32)
    q4 = r.integers(-3, 4, (2, 400, 2, 240)).astype(np.float32)
    cases.append(("quantized_240_k32_w32_P1600", q3, q4, 32, 32))
    g3 = r.standard_normal((3, 300, 2, 240)).astype(np.float32)
    g4 = r.standard_normal((3, 300, 2, 240)).astype(np.float32)
    cases.append(("gauss_240_k32_w32_P1800", g3, g4, 32, 32))
    # the wavefront kernel's top-64 sorts (k, budget <= 64) with dominance sets of
    # one, two and four registers, its full sorts (budget > 64), a budget below k,
    # and halves of 100 scores (two keys per lane)
    cases.append(("quantized_240_k48_w64_P1600", q3, q4, 48, 64))
    cases.append(("gauss_240_k64_w48_P1800", g3, g4, 64, 48))
    cases.append(("gauss_240_k8_w64_P1800", g3, g4, 8, 64))
    cases.append(("gauss_240_k33_w33_P1800", g3, g4, 33, 33))
    cases.append(("quantized_240_k16_w100_P1600", q3, q4, 16, 100))
    cases.append(("quantized_240_k32_w20_P1600", q3, q4, 32, 20))
    g5 = r.standard_normal((2, 300, 2, 100)).astype(np.float32)
    g6 = r.standard_normal((2, 300, 2, 100)).astype(np.float32)
    cases.append(("gauss_100_k32_w32_P1200", g5, g6, 32, 32))
    return cases


@pytest.mark.parametrize("case", _address_cases(), ids=lambda c: c[0])
def test_sdm_address_exact(case):
    name, s1, s2, k, budget = case
    announce(f"sdm_address {name} k={k} budget={budget} shape={s1.shape}")
    sslp = _sslp()
    idx, wt = sslp.sdm_address(torch.from_numpy(s1).to(DEV), torch.from_numpy(s2).to(DEV), k,
                               budget)
    torch.cuda.synchronize()
    ridx, rwt = oracle.sdm_address(s1, s2, k, budget)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(wt.cpu().numpy() - rwt).max() <= TOL_FP32
    # bf16 copy of the same scores ranks identically to the oracle on the bf16 values
    b1, b2 = torch.from_numpy(s1).bfloat16(), torch.from_numpy(s2).bfloat16()
    idx2, _ = sslp.sdm_address(b1.to(DEV), b2.to(DEV), k, budget)
    torch.cuda.synchronize()
    ridx2, _ = oracle.sdm_address(_np(b1), _np(b2), k, budget)
    np.testing.assert_array_equal(idx2.cpu().numpy(), ridx2)


def test_sparse_update_dense_limit_is_gdn():
    # every slot selected with raw weights wt_w = k_t, wt_r = q_t: the dense gated delta rule
    sslp = _sslp()
    announce("sdm_sparse_update dense limit vs GDN oracle")
    B, T, H, sq, dv = 2, 40, 2, 8, 12
    N = sq * sq
    g = torch.Generator().manual_seed(9)
    q = torch.randn((B, T, H, N), generator=g)
    k = torch.randn((B, T, H, N), generator=g)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((B, T, H, dv), generator=g)
    alpha = torch.empty((B, T, H)).uniform_(0.9, 1.0, generator=g)
    beta = torch.rand((B, T, H), generator=g)
    S0 = torch.randn((B, H, N, dv), generator=g)
    perm = torch.randperm(N, generator=g).int()
    idx = perm.expand(B, T, H, N).contiguous()
    wt_w = torch.gather(k, -1, idx.long()).contiguous()
    wt_r = torch.gather(q, -1, idx.long()).contiguous()
    M = S0.to(DEV).contiguous()
    y = sslp.sdm_sparse_update(idx.to(DEV), wt_w.to(DEV), idx.to(DEV), wt_r.to(DEV), v.to(DEV),
                               alpha.to(DEV), beta.to(DEV), M)
    torch.cuda.synchronize()
    S, o = oracle.gdn(q.numpy(), k.numpy(), v.numpy(), alpha.numpy(), beta.numpy(),
                      S0=S0.double().numpy())
    e_y, e_M = maxrel(y.cpu().double().numpy(), o, name="y"), maxrel(M.cpu().double().numpy(), S, name="M")
    print(f"  dense limit: y {e_y:.2e} M {e_M:.2e}", flush=True)
    assert e_y <= TOL_FP32 and e_M <= TOL_FP32


def test_decode_steps_equal_forward_and_chaining():
    sslp = _sslp()
    cfg = wl.SdmConfig("decode_small", 3, 12, 2, 16, 24, 6, 6, 9, 7, torch.bfloat16, 31)
    announce("decode steps == forward; forward(T1)+forward(T2) == forward(T1+T2)")
    x = wl.sdm_inputs(cfg)
    xd = {k: v.to(DEV) for k, v in x.items()}
    M0 = torch.randn((cfg.B, cfg.H, cfg.N, cfg.d_v), generator=torch.Generator().manual_seed(2))
    Mf = M0.to(DEV).contiguous()
    yf = sslp.sdm_forward(xd["sw1"], xd["sw2"], xd["sr1"], xd["sr2"], xd["v"], xd["alpha"],
                          xd["beta"], Mf, cfg.k_w, cfg.k_r, cfg.W, cfg.R)
    Md = M0.to(DEV).contiguous()
    ys = []
    for t in range(cfg.T):
        sl = {k: v[:, t].contiguous() for k, v in xd.items()}
        ys.append(sslp.sdm_decode_step(sl["sw1"], sl["sw2"], sl["sr1"], sl["sr2"], sl["v"],
                                       sl["alpha"], sl["beta"], Md, cfg.k_w, cfg.k_r, cfg.W,
                                       cfg.R))
    yd = torch.stack(ys, 1)
    Mc = M0.to(DEV).contiguous()
    T1 = 5
    part = [{k: v[:, a:b].contiguous() for k, v in xd.items()} for a, b in ((0, T1), (T1, cfg.T))]
    yc = [sslp.sdm_forward(p["sw1"], p["sw2"], p["sr1"], p["sr2"], p["v"], p["alpha"], p["beta"],
                           Mc, cfg.k_w, cfg.k_r, cfg.W, cfg.R) for p in part]
    torch.cuda.synchronize()
    assert maxrel(yd.cpu().float().numpy(), yf.cpu().float().numpy(), name="yd") <= 1e-6
    assert maxrel(Md.cpu().numpy(), Mf.cpu().numpy(), name="Md") <= 1e-6
    assert torch.equal(torch.cat(yc, 1).cpu(), yf.cpu())
    assert torch.equal(Mc.cpu(), Mf.cpu())


def test_decode_steps_replayed_from_a_graph_match_eager():
    # a serving loop captures its decode steps in a HIP graph and replays them;
    # every replay (the table reset eagerly in between, with synchronisations)
    # must give the eager steps' outputs and table bit for bit
    sslp = _sslp()
    cfg = wl.SdmConfig("decode_graph", 5, 4, 2, 20, 300, 8, 8, 16, 16, torch.bfloat16, 52)
    announce("decode steps: HIP graph replays == eager steps")
    x = {k: v.to(DEV) for k, v in wl.sdm_inputs(cfg).items()}
    sl = [{k: v[:, t].contiguous() for k, v in x.items()} for t in range(cfg.T)]
    M0 = torch.randn((cfg.B, cfg.H, cfg.N, cfg.d_v), generator=torch.Generator().manual_seed(5))
    M0 = M0.to(DEV)

    def steps(M, ys):
        for t, s in enumerate(sl):
            sslp.sdm_decode_step(s["sw1"], s["sw2"], s["sr1"], s["sr2"], s["v"], s["alpha"],
                                 s["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R, y=ys[t])

    Me = M0.clone()
    ye = [torch.empty((cfg.B, cfg.H, cfg.d_v), dtype=cfg.dtype, device=DEV) for _ in sl]
    steps(Me, ye)
    torch.cuda.synchronize()
    Mg = M0.clone()
    yg = [torch.empty_like(y) for y in ye]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps(Mg, yg)  # eager warm-up before the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(Mg, yg)
    for rep in range(3):
        Mg.copy_(M0)
        for y in yg:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Mg, Me), f"replay {rep}: table"
        for t in range(cfg.T):
            assert torch.equal(yg[t], ye[t]), f"replay {rep}: y of step {t}"


def test_repeatable_bitwise():
    sslp = _sslp()
    cfg = wl.SdmConfig("rep", 1, 64, 2, 64, 64, 16, 16, 32, 32, torch.bfloat16, 44)
    announce("bitwise repeatability")
    x = {k: v.to(DEV) for k, v in wl.sdm_inputs(cfg).items()}
    outs = []
    for _ in range(2):
        M = torch.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v), device=DEV)
        y = sslp.sdm_forward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"],
                             x["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R)
        outs.append((y.cpu(), M.cpu()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_empty_sequence_is_noop():
    sslp = _sslp()
    cfg = wl.SdmConfig("empty", 1, 0, 1, 8, 16, 4, 4, 4, 4, torch.float32, 1)
    x = {k: v.to(DEV) for k, v in wl.sdm_inputs(cfg).items()}
    M = torch.randn((1, 1, 64, 16), device=DEV)
    M0 = M.clone()
    sslp.sdm_forward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"], x["beta"], M,
                     4, 4, 4, 4)
    torch.cuda.synchronize()
    assert torch.equal(M, M0)


@pytest.mark.slow
@pytest.mark.parametrize("budget", [32, 64])
def test_sdm_1p4b_layer_full_size(budget):
    # the 1.4B-layer prefill at k = W = R = 32 (16-token chunks) and at the
    # pages' larger budget k = W = R = 64 (8-token chunks)
    cfg = dataclasses.replace(wl.SDM_14B, k_w=budget, k_r=budget, W=budget, R=budget)
    announce(f"sdm 1.4B-layer full size T={cfg.T} N={cfg.N} d_v={cfg.d_v} W=R={budget}")
    x = wl.sdm_inputs(cfg)
    M0 = torch.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v))
    got = _run_forward(cfg, x, M0, 0)
    ref = _oracle_forward(cfg, x, M0, 0)
    _check(cfg, got, ref, M0, "1.4B layer")


@pytest.mark.slow
@pytest.mark.parametrize("sqrt_n", [362, 363])
def test_sdm_row_offsets_at_the_32_bit_limit(sqrt_n):
    # the largest tables d_v allows (4096 columns): 362^2 slots keep every row
    # offset below 2^31 bytes (the chunk path's 32-bit offsets, the largest
    # ones it takes), 363^2 slots cross it (the per-token path, 64-bit offsets)
    cfg = wl.SdmConfig("offsets", 1, 64, 1, sqrt_n, 4096, 32, 32, 32, 32, torch.bfloat16,
                       800 + sqrt_n)
    announce(f"sdm table of {cfg.N} x 4096 fp32 ({cfg.N * 4096 * 4 / 2**31:.4f} x 2^31 bytes)")
    x = wl.sdm_inputs(cfg)
    M0 = torch.zeros((1, 1, cfg.N, cfg.d_v))
    got = _run_forward(cfg, x, M0, 0)
    ref = _oracle_forward(cfg, x, M0, 0)
    assert int(ref["idx_w"].max()) * 4096 * 4 > 2**31 - 2**24  # rows near the end were written
    _check(cfg, got, ref, M0, f"offsets sqrtN={sqrt_n}")


@pytest.mark.slow
def test_sdm_1p4b_layer_batch8_sampled():
    # the batch-8 row of the benchmark (1,920 column slices: the chunk path
    # runs them in rounds), all eight sequences in one call; sequences are
    # independent, so the oracle checks the first and the last one
    cfg = dataclasses.replace(wl.SDM_14B, B=8)
    announce(f"sdm 1.4B-layer B=8 T={cfg.T}, sequences 0 and 7 checked")
    x = wl.sdm_inputs(cfg)
    M0 = torch.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v))
    got = _run_forward(cfg, x, M0, 0)
    sub = [0, cfg.B - 1]
    c2 = dataclasses.replace(cfg, B=len(sub))
    xs = {k: v[sub] for k, v in x.items()}
    ref = _oracle_forward(c2, xs, M0[sub], 0)
    gs = dict(y=got["y"][sub], M=got["M"][sub], idx_w=got["idx_w"][sub], wt_w=got["wt_w"][sub],
              idx_r=got["idx_r"][sub], wt_r=got["wt_r"][sub])
    _check(c2, gs, ref, M0[sub], "1.4B layer, B=8 (sequences 0, 7)")


@pytest.mark.slow
def test_sdm_decode_full_size():
    # 64 independent sequences on the 1.4B-layer table shape (28.3 GB state).  The
    # pre-step table is drawn by torch on the device; the oracle recomputes the
    # addressing and the step from copies of the rows it selects.
    sslp = _sslp()
    cfg = wl.SDM_DECODE
    announce(f"sdm decode full size B={cfg.B} H={cfg.H} N={cfg.N} d_v={cfg.d_v}")
    g = torch.Generator(device=DEV).manual_seed(cfg.seed)
    M = torch.empty((cfg.B, cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device=DEV)
    M.normal_(generator=g)
    x = wl.sdm_inputs(cfg)
    step = {k: v[:, 0].contiguous() for k, v in x.items()}
    n = {k: _np(v) for k, v in step.items()}
    idx_w, wt_w = oracle.sdm_address(n["sw1"], n["sw2"], cfg.k_w, cfg.W)  # [B,H,W]
    idx_r, wt_r = oracle.sdm_address(n["sr1"], n["sr2"], cfg.k_r, cfg.R)
    rows = np.concatenate([idx_w, idx_r], -1)  # [B,H,W+R]
    U = rows.shape[-1]
    # compact per-(b,h) tables holding only the touched rows, copied before the step
    rows_t = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    pre = torch.gather(M, 2, rows_t[..., None].expand(-1, -1, -1, cfg.d_v)).cpu().double().numpy()
    rng = np.random.default_rng(0)
    sample = rng.integers(0, cfg.N, (cfg.B, cfg.H, 16))
    sample_t = torch.from_numpy(sample).to(DEV)
    before = torch.gather(M, 2, sample_t[..., None].expand(-1, -1, -1, cfg.d_v)).cpu()
    # local slot ids inside the compact table: first occurrence of each slot
    loc = np.zeros_like(rows)
    for b in range(cfg.B):
        for h in range(cfg.H):
            first = {}
            for u in range(U):
                first.setdefault(int(rows[b, h, u]), u)
                loc[b, h, u] = first[int(rows[b, h, u])]
    lw = loc[..., :cfg.W][:, None].astype(np.int32)
    lr = loc[..., cfg.W:][:, None].astype(np.int32)
    Mref, yref = oracle.sdm_recurrence(lw, wt_w[:, None], lr, wt_r[:, None], n["v"][:, None],
                                       n["alpha"][:, None], n["beta"][:, None], pre,
                                       residual_mode=0)
    sd = {k: v.to(DEV) for k, v in step.items()}
    iw = torch.empty((cfg.B, cfg.H, cfg.W), dtype=torch.int32, device=DEV)
    ir = torch.empty((cfg.B, cfg.H, cfg.R), dtype=torch.int32, device=DEV)
    y = sslp.sdm_decode_step(sd["sw1"], sd["sw2"], sd["sr1"], sd["sr2"], sd["v"], sd["alpha"],
                             sd["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R, idx_w=iw, idx_r=ir)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(iw.cpu().numpy(), idx_w)
    np.testing.assert_array_equal(ir.cpu().numpy(), idx_r)
    post = torch.gather(M, 2, rows_t[..., None].expand(-1, -1, -1, cfg.d_v)).cpu().double().numpy()
    # rows of the compact reference in the same order as `rows`
    Mrows = np.take_along_axis(Mref, loc[..., None].astype(np.int64), axis=2)
    e_y = maxrel(y.cpu().double().numpy(), yref[:, 0], name="y")
    e_M = maxrel(post, Mrows, name="M_rows")
    print(f"  decode full: y {e_y:.2e} M rows {e_M:.2e}", flush=True)
    assert e_y <= TOL_BF16 and e_M <= TOL_FP32
    after = torch.gather(M, 2, sample_t[..., None].expand(-1, -1, -1, cfg.d_v)).cpu()
    touched = np.array([[np.isin(sample[b, h], idx_w[b, h]) for h in range(cfg.H)]
                        for b in range(cfg.B)])
    assert torch.equal(after[torch.from_numpy(~touched)], before[torch.from_numpy(~touched)])
    del M
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,W", [(48, 16), (80, 32)])
def test_forward_equals_component_calls(T, W):
    # sdm_forward is the kernel sequence write-addressing, read-addressing,
    # recurrence; the benchmark issues the same sequence through the component
    # entry points to time the recurrence on its own
    sslp = _sslp()
    cfg = wl.SdmConfig("compose", 1, T, 2, 32, 40, 8, 8, W, W, torch.bfloat16, 55)
    announce("sdm_forward == sdm_address x2 + sdm_sparse_update")
    x = {k: v.to(DEV) for k, v in wl.sdm_inputs(cfg).items()}
    M1 = torch.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v), device=DEV)
    M2 = torch.zeros_like(M1)
    y1 = sslp.sdm_forward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"], x["beta"],
                          M1, cfg.k_w, cfg.k_r, cfg.W, cfg.R)
    iw, ww = sslp.sdm_address(x["sw1"], x["sw2"], cfg.k_w, cfg.W)
    ir, wr = sslp.sdm_address(x["sr1"], x["sr2"], cfg.k_r, cfg.R)
    y2 = sslp.sdm_sparse_update(iw, ww, ir, wr, x["v"], x["alpha"], x["beta"], M2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(M1, M2)


def test_side_stream_call_orders_its_own_allocations():
    # sdm_forward enqueued on a stream other than the current one, with the
    # binding's own workspace and output; the current stream then allocates and
    # fills memory at once.  The binding allocates on the call's stream, so
    # nothing it still uses can be handed out meanwhile: results equal a plain
    # call on the current stream, bit for bit.
    sslp = _sslp()
    cfg = wl.SdmConfig("side", 1, 200, 2, 64, 64, 16, 16, 32, 32, torch.bfloat16, 66)
    announce("sdm_forward on a side stream, allocations on the current stream meanwhile")
    x = {k: v.to(DEV) for k, v in wl.sdm_inputs(cfg).items()}
    M_ref = torch.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v), device=DEV)
    y_ref = sslp.sdm_forward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"],
                             x["beta"], M_ref, cfg.k_w, cfg.k_r, cfg.W, cfg.R)
    M = torch.zeros_like(M_ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    y = sslp.sdm_forward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"], x["beta"],
                         M, cfg.k_w, cfg.k_r, cfg.W, cfg.R, stream=side)
    junk = [torch.full((1 << 22,), float("nan"), device=DEV) for _ in range(16)]
    torch.cuda.synchronize()
    del junk
    assert torch.equal(y, y_ref) and torch.equal(M, M_ref)


@pytest.mark.parametrize("path", ["chunked", "chunked_w64", "per_token"])
def test_out_of_range_slot_is_contained_and_reported(path):
    # A caller index outside [0, N) must not reach memory outside the table: the
    # table is a slice of a larger buffer whose guard regions must stay bitwise;
    # the device error flag reports the call.  Chunk path: W = R = 32 or 64,
    # T >= 64; per-token path: W = R = 9.
    sslp = _sslp()
    W = {"chunked": 32, "chunked_w64": 64, "per_token": 9}[path]
    B, T, H, sq, dv = 1, 80, 2, 16, 32
    N = sq * sq
    announce(f"out-of-range slot, {path} path")
    assert not sslp.device_error()  # clear anything left over
    g = torch.Generator().manual_seed(91)
    idx = torch.stack([torch.randperm(N, generator=g)[:W] for _ in range(B * T * H)]).int()
    idx = idx.view(B, T, H, W).contiguous()
    idx[0, 70, 1, 3] = N + 5           # one bad write slot (token 70, head 1)
    idx_r = idx.clone()
    idx_r[0, 10, 0, 0] = -7            # one bad read slot (token 10, head 0)
    wt = torch.full((B, T, H, W), 1.0 / W)
    v = torch.randn((B, T, H, dv), generator=g)
    alpha = torch.full((B, T, H), 0.95)
    beta = torch.full((B, T, H), 0.5)
    guard = 1 << 16
    buf = torch.randn((2 * guard + B * H * N * dv,), generator=g).to(DEV)
    before = buf.clone()
    M = buf[guard:guard + B * H * N * dv].view(B, H, N, dv)
    y = sslp.sdm_sparse_update(idx.to(DEV), wt.to(DEV), idx_r.to(DEV), wt.to(DEV), v.to(DEV),
                               alpha.to(DEV), beta.to(DEV), M)
    torch.cuda.synchronize()
    assert sslp.device_error()
    assert not sslp.device_error()  # the query cleared it
    assert torch.equal(buf[:guard], before[:guard])
    assert torch.equal(buf[-guard:], before[-guard:])
    assert torch.isfinite(y).all()
    # a clean call after it reports nothing
    idx[0, 70, 1, 3] = 0 if 0 not in idx[0, 70, 1].tolist() else int(
        [s for s in range(N) if s not in idx[0, 70, 1].tolist()][0])
    sslp.sdm_sparse_update(idx.to(DEV), wt.to(DEV), idx.to(DEV), wt.to(DEV), v.to(DEV),
                           alpha.to(DEV), beta.to(DEV), M)
    assert not sslp.device_error()
