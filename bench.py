"""Benchmark of the sparse-routed gated delta-rule hot path on one MI355X.

Default workload: one Sparse Delta Memory layer at the 1.4B-layer shape
(B=1, T=8192, H=2, N=57,600 slots of d_v=960, per-half top-32, W=R=32, bf16
inputs, fp32 table).  One step = write addressing + read addressing + the
sparse decay/update/read recurrence over all 8192 tokens (the kernel sequence
of sdm_forward, issued through its component entry points so that the
recurrence kernel can be timed on its own with HIP events).

Prints ONE JSON line (see the keys below).  `value` is tokens/s of the whole
step; `roofline` reports the dominant kernel (the recurrence) against HBM
bandwidth using the algorithmic bytes it must move; `cpu_baseline` times the
fp64 oracle on the host.
"""
import argparse
import dataclasses
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
SDM_SRC = os.path.join(ROOT, "sparse_state_linear_product_amd", "csrc", "sdm_chunk.hip")
SDM_PROFILE = os.path.join(ROOT, "profiles", "sdm_chunk_apply_1p4b_prefill.md")


def measured_traffic(src=SDM_SRC, profile=SDM_PROFILE):
    """HBM bytes per launch from the committed counter summary, or None.

    The summary records the scaled FETCH_SIZE + WRITE_SIZE bytes of one
    sdm_sparse_update launch (plan + apply kernels) together with the sha256 of
    the kernel source it was taken on; once the source changes the counters no
    longer describe the kernel and the figure is withheld.
    """
    import hashlib
    try:
        text = open(profile).read()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    m_s = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not (m_b and m_s) or m_s.group(1) != sha:
        return None
    return int(m_b.group(1))


def sdm_kernel_bytes(cfg, io_bytes):
    """Algorithmic bytes the recurrence kernel moves per launch.

    Per (token, head): W rows gathered + W rows scattered + R rows gathered of
    d_v fp32 = (2W+R)*d_v*4; v read and y written (d_v each, io dtype); alpha,
    beta (8 B); the write/read slot lists and weights (W+R)*8.
    """
    per = (2 * cfg.W + cfg.R) * cfg.d_v * 4 + 2 * cfg.d_v * io_bytes + 8 + (cfg.W + cfg.R) * 8
    return per * cfg.B * cfg.T * cfg.H, per


def bench_sdm(args, torch, sslp, wl):
    cfg = wl.SDM_14B
    dev = torch.device("cuda:0")
    x = {k: v.to(dev) for k, v in wl.sdm_inputs(cfg).items()}
    M = torch.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device=dev)
    shp = (cfg.B, cfg.T, cfg.H)
    iw = torch.empty(shp + (cfg.W,), dtype=torch.int32, device=dev)
    ww = torch.empty(shp + (cfg.W,), dtype=torch.float32, device=dev)
    ir = torch.empty(shp + (cfg.R,), dtype=torch.int32, device=dev)
    wr = torch.empty(shp + (cfg.R,), dtype=torch.float32, device=dev)
    y = torch.empty(shp + (cfg.d_v,), dtype=cfg.dtype, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        sslp.sdm_address(x["sw1"], x["sw2"], cfg.k_w, cfg.W, idx=iw, wt=ww)
        sslp.sdm_address(x["sr1"], x["sr2"], cfg.k_r, cfg.R, idx=ir, wt=wr)
        if ev is not None:
            ev[0].record(stream)
        sslp.sdm_sparse_update(iw, ww, ir, wr, x["v"], x["alpha"], x["beta"], M, y=y)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    k_ms = [a.elapsed_time(b) for a, b in evs]
    k_avg_ms = sum(k_ms) / len(k_ms)
    nbytes, per = sdm_kernel_bytes(cfg, 2 if cfg.dtype == torch.bfloat16 else 4)
    achieved = nbytes / (k_avg_ms * 1e-3) / 1e9
    tokens = cfg.B * cfg.T * args.steps
    return dict(
        cfg=cfg, ms_per_step=total_ms / args.steps, value=tokens / (total_ms * 1e-3),
        roofline=dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(),
                      kernel="sdm_sparse_update: sdm_chunk_plan_kernel + sdm_chunk_apply_kernel",
                      kernel_avg_ms=round(k_avg_ms, 4),
                      bytes_per_launch=nbytes, bytes_per_token_head=per))


def time_call(torch, fn, reps, warmup=2):
    """Average milliseconds of fn() on the current stream (HIP events)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_graph(torch, fn, reps, warmup=1):
    """Average milliseconds of one replay of a HIP graph that holds fn()'s launches.

    A serving loop replays a captured decode step instead of issuing its
    launches from Python one by one; this times the GPU side of that loop.
    fn() runs once eagerly (on a side stream) before the capture.
    """
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / reps


BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def gdn_flops(B, T, H, dk, dv, C=64):
    """Lean chunked-WY FLOP count per call: 2*(2C*dk + 1.5C*dv + 3*dk*dv) per token-head."""
    return 2 * (2 * C * dk + 1.5 * C * dv + 3 * dk * dv) * B * T * H


def gdn_bytes(B, T, H, dk, dv, kda):
    """q, k, v bf16 in; o bf16 out; alpha (per token or per channel) and beta fp32; state out."""
    per = 2 * (2 * dk + dv) + 2 * dv + 4 * (dk if kda else 1) + 4
    return per * B * T * H + 4 * B * H * dk * dv


def bench_rows(args, torch, sslp, wl):
    rows = {}
    dev = torch.device("cuda:0")
    for cfg in (wl.GDN, wl.KDA):
        x = {k: v.to(dev) for k, v in wl.gdn_inputs(cfg).items()}
        o = torch.empty_like(x["v"])
        S = torch.empty((cfg.B, cfg.H, cfg.d_k, cfg.d_v), dtype=torch.float32, device=dev)
        ms = time_call(torch, lambda: sslp.gdn_chunk_forward(x["q"], x["k"], x["v"], x["alpha"],
                                                             x["beta"], S_out=S, o=o), args.steps)
        fl = gdn_flops(cfg.B, cfg.T, cfg.H, cfg.d_k, cfg.d_v)
        by = gdn_bytes(cfg.B, cfg.T, cfg.H, cfg.d_k, cfg.d_v, cfg.kda)
        rows[cfg.name] = dict(ms=round(ms, 4), tokens_per_s=round(cfg.B * cfg.T / (ms * 1e-3), 1),
                              tflops=round(fl / (ms * 1e-3) / 1e12, 2),
                              mfma_frac=round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                              gbs=round(by / (ms * 1e-3) / 1e9, 1),
                              hbm_frac=round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              flops_per_call=fl, bytes_per_call=by)
        del x, o, S
    # GDN2: KDA decay, erase vector b [d_k] and write vector w [d_v] per token in place of beta
    cfg = wl.GDN2
    x = {k: v.to(dev) for k, v in wl.gdn2_inputs(cfg).items()}
    o = torch.empty_like(x["v"])
    S = torch.empty((cfg.B, cfg.H, cfg.d_k, cfg.d_v), dtype=torch.float32, device=dev)
    ms = time_call(torch, lambda: sslp.gdn2_chunk_forward(x["q"], x["k"], x["v"], x["alpha"],
                                                          x["erase"], x["write"], S_out=S, o=o),
                   args.steps)
    fl = gdn_flops(cfg.B, cfg.T, cfg.H, cfg.d_k, cfg.d_v)
    by = gdn_bytes(cfg.B, cfg.T, cfg.H, cfg.d_k, cfg.d_v, True) + 4 * (cfg.d_k + cfg.d_v - 1) * cfg.B * cfg.T * cfg.H
    rows[cfg.name] = dict(ms=round(ms, 4), tokens_per_s=round(cfg.B * cfg.T / (ms * 1e-3), 1),
                          tflops=round(fl / (ms * 1e-3) / 1e12, 2),
                          mfma_frac=round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                          gbs=round(by / (ms * 1e-3) / 1e9, 1),
                          hbm_frac=round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          flops_per_call=fl, bytes_per_call=by)
    del x, o, S
    # SSE: B=4, T=4096, H=16, 8 routed + 1 shared partition, top-2, c=d=128
    cfg = wl.SSE
    x = {k: v.to(dev) for k, v in wl.sse_inputs(cfg).items()}
    S = torch.zeros((cfg.B, cfg.H, cfg.N + 1, cfg.c, cfg.d), dtype=torch.float32, device=dev)
    o = torch.empty_like(x["v"])
    ms = time_call(torch, lambda: sslp.sse_forward(x["logits"], x["q"], x["k"], x["v"], x["lam"],
                                                   S, cfg.topk, o=o), args.steps)
    per = 2 * (2 * cfg.c + cfg.d) + 4 * cfg.c + 4 * cfg.N + 2 * cfg.d
    by = per * cfg.B * cfg.T * cfg.H + 2 * 4 * cfg.B * cfg.H * (cfg.N + 1) * cfg.c * cfg.d
    rows[cfg.name] = dict(ms=round(ms, 4), tokens_per_s=round(cfg.B * cfg.T / (ms * 1e-3), 1),
                          gbs=round(by / (ms * 1e-3) / 1e9, 1),
                          hbm_frac=round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          bytes_per_call=by)
    # the same workload as the masking execution (every partition steps over every token)
    ms = time_call(torch, lambda: sslp.sse_forward(x["logits"], x["q"], x["k"], x["v"], x["lam"],
                                                   S, cfg.topk, o=o, masking=True), args.steps)
    rows[cfg.name + "_masking"] = dict(ms=round(ms, 4),
                                       tokens_per_s=round(cfg.B * cfg.T / (ms * 1e-3), 1),
                                       gbs=round(by / (ms * 1e-3) / 1e9, 1),
                                       hbm_frac=round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                       bytes_per_call=by)
    del x, S, o
    # SSE grouped (varlen) against masked execution over sequence lengths, the
    # comparison of the SSE slides' Fig. 6 (there: fwd+bwd on another GPU; here
    # the forward): B=4, H=16, c=d=128, N routed partitions, top-k
    sweep = {}
    for N, topk in ((4, 1), (8, 1), (8, 2)):
        for T in (256, 1024, 4096):
            c2 = dataclasses.replace(wl.SSE, N=N, topk=topk, T=T)
            x = {k: v.to(dev) for k, v in wl.sse_inputs(c2).items()}
            S = torch.zeros((c2.B, c2.H, N + 1, c2.c, c2.d), dtype=torch.float32, device=dev)
            o = torch.empty_like(x["v"])
            reps = max(3, args.steps)
            t_var = time_call(torch, lambda: sslp.sse_forward(x["logits"], x["q"], x["k"], x["v"],
                                                              x["lam"], S, topk, o=o), reps)
            t_msk = time_call(torch, lambda: sslp.sse_forward(x["logits"], x["q"], x["k"], x["v"],
                                                              x["lam"], S, topk, o=o, masking=True),
                              reps)
            sweep[f"N{N}_k{topk}_T{T}"] = dict(varlen_ms=round(t_var, 4), masking_ms=round(t_msk, 4))
            del x, S, o
    rows["sse_masking_vs_varlen_B4_H16_c128"] = sweep
    # SSE decode: 64 independent sequences, N=8 routed + 1 shared states of 128x128 per head;
    # a step reads and writes the 2 selected and the shared state of every (sequence, head)
    cfg = wl.SSE_DECODE
    S = torch.empty((cfg.B, cfg.H, cfg.N + 1, cfg.c, cfg.d), dtype=torch.float32, device=dev)
    S.normal_(generator=torch.Generator(device=dev).manual_seed(cfg.seed))
    steps = {k: v.to(dev) for k, v in wl.sse_inputs(cfg, T=args.decode_steps).items()}
    sl = [{k: v[:, t].contiguous() for k, v in steps.items()} for t in range(args.decode_steps)]
    o = torch.empty((cfg.B, cfg.H, cfg.d), dtype=cfg.dtype, device=dev)

    def sse_steps():
        for s in sl:
            sslp.sse_decode_step(s["logits"], s["q"], s["k"], s["v"], s["lam"], S, cfg.topk, o=o)

    ms = time_call(torch, sse_steps, 1, warmup=1) / args.decode_steps
    per = 2 * (cfg.topk + 1) * cfg.c * cfg.d * 4 + 4 * cfg.N + 2 * (2 * cfg.c + cfg.d) + 4 * cfg.c + 2 * cfg.d
    nbytes = per * cfg.B * cfg.H
    rows[cfg.name] = dict(ms_per_step=round(ms, 4), tokens_per_s=round(cfg.B / (ms * 1e-3), 1),
                          gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                          hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          bytes_per_step=nbytes, steps=args.decode_steps)
    del S, steps, sl, o
    # SDM decode: 64 independent sequences on the 1.4B-layer table shape
    cfg = wl.SDM_DECODE
    M = torch.empty((cfg.B, cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device=dev)
    M.normal_(generator=torch.Generator(device=dev).manual_seed(cfg.seed))
    pre = wl.sdm_inputs(cfg, T=wl.DECODE_PREFIX, seed=cfg.seed + 1)
    pre = {k: v.to(dev) for k, v in pre.items()}
    sslp.sdm_forward(pre["sw1"], pre["sw2"], pre["sr1"], pre["sr2"], pre["v"], pre["alpha"],
                     pre["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R)
    del pre
    steps = {k: v.to(dev) for k, v in wl.sdm_inputs(cfg, T=args.decode_steps).items()}
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    y = torch.empty((cfg.B, cfg.H, cfg.d_v), dtype=cfg.dtype, device=dev)
    sl = [{k: v[:, t].contiguous() for k, v in steps.items()} for t in range(args.decode_steps)]

    def run_steps():
        for s in sl:
            sslp.sdm_decode_step(s["sw1"], s["sw2"], s["sr1"], s["sr2"], s["v"], s["alpha"],
                                 s["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R, y=y, workspace=ws)

    ms_eager = time_call(torch, run_steps, 1, warmup=1) / args.decode_steps
    # the same steps replayed from a HIP graph: the launches no longer wait on
    # the Python binding, so this is the GPU's own rate
    ms = time_graph(torch, run_steps, 3) / args.decode_steps
    nbytes, per = sdm_kernel_bytes(cfg, 2)
    nbytes = per * cfg.B * cfg.H
    rows[cfg.name] = dict(ms_per_step=round(ms, 4), ms_per_step_eager=round(ms_eager, 4),
                          tokens_per_s=round(cfg.B / (ms * 1e-3), 1),
                          gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                          hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          bytes_per_step=nbytes, steps=args.decode_steps)
    del M
    torch.cuda.empty_cache()
    # the 1.4B prefill layer at batch 8 (1,920 column slices: the chunk-parallel
    # path runs them in rounds) and at the pages' W = R = 64 budget (chunks of 8
    # tokens), each as one sdm_forward call (addressing + update)
    for tag, c2 in (("B8", dataclasses.replace(wl.SDM_14B, B=8)),
                    ("W64_k64", dataclasses.replace(wl.SDM_14B, k_w=64, k_r=64, W=64, R=64))):
        x = {k: v.to(dev) for k, v in wl.sdm_inputs(c2).items()}
        M = torch.zeros((c2.B, c2.H, c2.N, c2.d_v), dtype=torch.float32, device=dev)
        y = torch.empty_like(x["v"])
        ms = time_call(torch, lambda: sslp.sdm_forward(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"],
                                                       x["alpha"], x["beta"], M, c2.k_w, c2.k_r,
                                                       c2.W, c2.R, y=y), 2, warmup=1)
        nbytes, _ = sdm_kernel_bytes(c2, 2)
        rows[f"sdm_prefill_1p4b_{tag}_T8192_H2_N57600_dv960"] = dict(
            ms=round(ms, 4), tokens_per_s=round(c2.B * c2.T / (ms * 1e-3), 1),
            gbs_forward=round(nbytes / (ms * 1e-3) / 1e9, 1),
            path=f"chunk-parallel, {16 if c2.W == 32 else 8}-token chunks")
        del x, M, y
        torch.cuda.empty_cache()
    # read epilogue (RMS-Norm + SiLU output gate) on the 1.4B prefill read y [1,8192,2,960] bf16
    cfg = wl.SDM_14B
    gen = torch.Generator(device=dev).manual_seed(cfg.seed + 9)
    yv = torch.randn((cfg.B, cfg.T, cfg.H, cfg.d_v), generator=gen, device=dev).to(cfg.dtype)
    gv = torch.randn(yv.shape, generator=gen, device=dev).to(cfg.dtype)
    gam = torch.rand((cfg.d_v,), generator=gen, device=dev) + 0.5
    ov = torch.empty_like(yv)
    ms = time_call(torch, lambda: sslp.sdm_norm_gate(yv, gam, gv, act="silu", o=ov), args.steps)
    nbytes = 3 * yv.numel() * 2 + cfg.d_v * 4
    rows["sdm_norm_gate_1p4b_T8192_H2_dv960"] = dict(
        ms=round(ms, 4), gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
        hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), bytes_per_call=nbytes)
    del yv, gv, gam, ov
    # SDM training on the 1.4B prefill layer: forward keeping the pre-write rows
    # and the backward by undoing writes (both chunk-parallel; the backward's
    # slice reduction and addressing-softmax backward included)
    cfg = wl.SDM_14B
    x = {k: v.to(dev) for k, v in wl.sdm_inputs(cfg).items()}
    M = torch.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v), dtype=torch.float32, device=dev)
    y, ctx = sslp.sdm_forward_train(x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"],
                                    x["beta"], M, cfg.k_w, cfg.k_r, cfg.W, cfg.R)
    dy = torch.randn(y.shape, device=dev).to(cfg.dtype)
    dM = torch.zeros_like(M)
    ws = torch.empty(sslp.sdm_backward_workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.sqrtN, cfg.d_v,
                                                       cfg.W, cfg.R), dtype=torch.uint8,
                     device=dev)
    ws_f = torch.empty(max(1, sslp.sdm_train_workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.sqrtN,
                                                             cfg.d_v, cfg.W, cfg.R)),
                       dtype=torch.uint8, device=dev)
    reps = max(2, args.steps // 5)
    ms_f = time_call(torch, lambda: sslp.sdm_forward_train(
        x["sw1"], x["sw2"], x["sr1"], x["sr2"], x["v"], x["alpha"], x["beta"], M, cfg.k_w,
        cfg.k_r, cfg.W, cfg.R, y=y, out=ctx, workspace=ws_f), reps, warmup=1)
    ms_b = time_call(torch, lambda: sslp.sdm_backward(ctx, x["v"], x["alpha"], x["beta"], M, dy,
                                                      dM, workspace=ws), reps, warmup=1)
    ntok = cfg.B * cfg.T * cfg.H
    _, per_f = sdm_kernel_bytes(cfg, 2)
    per_f += cfg.W * cfg.d_v * 4
    per_b = (3 * cfg.R + 4 * cfg.W) * cfg.d_v * 4 + 3 * cfg.d_v * 2 + 8 + (cfg.W + cfg.R) * 8
    rows["sdm_train_" + cfg.name.split("sdm_prefill_")[-1]] = dict(
        fwd_ms=round(ms_f, 4), bwd_ms=round(ms_b, 4),
        tokens_per_s=round(cfg.B * cfg.T / ((ms_f + ms_b) * 1e-3), 1),
        fwd_gbs=round(per_f * ntok / (ms_f * 1e-3) / 1e9, 1),
        fwd_hbm_frac=round(per_f * ntok / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        bwd_gbs=round(per_b * ntok / (ms_b * 1e-3) / 1e9, 1),
        bwd_hbm_frac=round(per_b * ntok / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        fwd_bytes_per_token_head=per_f, bwd_bytes_per_token_head=per_b)
    del x, M, y, ctx, dy, dM, ws, ws_f
    torch.cuda.empty_cache()
    return rows


def cpu_baseline_sdm(wl, torch):
    import numpy as np

    import oracle

    cfg = wl.SDM_14B
    x = wl.sdm_inputs(cfg)
    n = {k: wl.to_numpy_f32(v) for k, v in x.items()}
    M0 = np.zeros((cfg.B, cfg.H, cfg.N, cfg.d_v))
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.sdm_forward(n["sw1"], n["sw2"], n["sr1"], n["sr2"], n["v"], n["alpha"], n["beta"],
                           M0, cfg.k_w, cfg.k_r, cfg.W, cfg.R)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or reps >= 20:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    # the addressing runs one problem per thread over all threads; the recurrence
    # runs one (b, h, 64-column block) unit per thread
    units = cfg.B * cfg.H * -(-cfg.d_v // 64)
    used = min(threads, units)
    return dict(value=round(cfg.B * cfg.T * reps / el, 1), unit="tokens/s", cores=used,
                kind="oracle",
                sample=f"full workload ({cfg.B * cfg.T} tokens x {cfg.H} heads) repeated {reps}x, "
                       f"{el:.1f} s; fp64 C/OpenMP oracle on {used} threads (addressing: one "
                       f"problem per thread; recurrence: {units} (b, h, 64-column) units)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the other hot-path rows")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device copy, the reference dispatch for "
                         "scaling hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the per-GPU shard is the single-GPU workload", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_state_linear_product_amd as sslp
    from sparse_state_linear_product_amd import workloads as wl

    if args.calibrate_copy:
        n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    r = bench_sdm(args, torch, sslp, wl)
    cfg = r["cfg"]
    out = {
        "metric": "tokens/s per layer + achieved HBM GB/s (sparse update), % roofline, 1 MI355X",
        "value": round(r["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "H": cfg.H, "N": cfg.N,
                   "d_v": cfg.d_v, "k": cfg.k_w, "W": cfg.W, "R": cfg.R, "inputs": "bf16",
                   "state": "fp32", "residual": "shared"},
        "roofline": r["roofline"],
    }
    if not args.no_rows:
        out["rows"] = bench_rows(args, torch, sslp, wl)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_sdm(wl, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
