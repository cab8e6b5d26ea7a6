"""Seeded synthetic workloads with the shapes and value distributions of the
pages' configurations.

Input generation only: nothing here computes any step of the method.  Every
tensor is drawn on the CPU from a torch.Generator seeded per configuration,
in the fixed order written in each function, and rounded once to the stated
dtype; the oracle reads exactly these rounded values (bf16 -> fp32 is exact).

Distributions (the pages give the shapes; the gate means follow the Sparse
Delta Memory slides' probe, forget gate ~0.95 and input gate ~0.50, which
U(0.9,1) and U(0,1) reproduce):
  SDM  score halves, v ~ N(0,1); alpha ~ U(0.9,1), beta ~ U(0,1) per (b,t,h)
  GDN  q, v ~ N(0,1); k = g/|g|_2 with g ~ N(0,1) (normalised in fp32, then
       rounded); beta = sigmoid(N(0,1)); alpha ~ U(0.9,1) per (b,t,h) or per
       (b,t,h,channel)
  SSE  logits ~ N(0,1) fp32; k = softmax over c of N(0,1) logits; q, v ~ N(0,1);
       lambda ~ U(0.95,1) per (b,t,h,row)
"""
from dataclasses import dataclass

import torch

BF16 = torch.bfloat16
F32 = torch.float32


@dataclass(frozen=True)
class SdmConfig:
    name: str
    B: int
    T: int
    H: int
    sqrtN: int
    d_v: int
    k_w: int
    k_r: int
    W: int
    R: int
    dtype: torch.dtype
    seed: int

    @property
    def N(self):
        return self.sqrtN * self.sqrtN


@dataclass(frozen=True)
class GdnConfig:
    name: str
    B: int
    T: int
    H: int
    d_k: int
    d_v: int
    dtype: torch.dtype
    kda: bool
    seed: int


@dataclass(frozen=True)
class SseConfig:
    name: str
    B: int
    T: int
    H: int
    N: int
    topk: int
    c: int
    d: int
    dtype: torch.dtype
    seed: int


# The five configurations: SDM tiny fp32; dense GDN and KDA; SSE; SDM at the
# 1.4B-layer shape (d=1920, H=2 -> N=(d/4H)^2=57,600, d_v=d/H=960); SDM decode
# at that shape for 64 independent sequences.
SDM_TINY = SdmConfig("sdm_tiny_fp32", 1, 256, 1, 8, 16, 4, 4, 4, 4, F32, 1001)
GDN = GdnConfig("gdn_chunk_B4_T4096_H16_d128", 4, 4096, 16, 128, 128, BF16, False, 1002)
KDA = GdnConfig("kda_chunk_B4_T4096_H16_d128", 4, 4096, 16, 128, 128, BF16, True, 1012)
GDN2 = GdnConfig("gdn2_chunk_B4_T4096_H16_d128", 4, 4096, 16, 128, 128, BF16, True, 1014)
SSE = SseConfig("sse_B4_T4096_H16_N8k2_c128", 4, 4096, 16, 8, 2, 128, 128, BF16, 1003)
SDM_14B = SdmConfig("sdm_prefill_1p4b_B1_T8192_H2_N57600_dv960", 1, 8192, 2, 240, 960, 32, 32, 32,
                    32, BF16, 1004)
SDM_DECODE = SdmConfig("sdm_decode_1p4b_seq64_H2_N57600_dv960", 64, 1, 2, 240, 960, 32, 32, 32, 32,
                       BF16, 1005)
# SSE decode: 64 independent sequences, one token each per step, at the SSE layer shape
SSE_DECODE = SseConfig("sse_decode_seq64_H16_N8k2_c128", 64, 1, 16, 8, 2, 128, 128, BF16, 1013)
DECODE_PREFIX = 256  # tokens of seeded prefix written into each decode table by the benchmark


def _gen(seed):
    return torch.Generator().manual_seed(int(seed))


def _normal(shape, g, dtype):
    return torch.randn(shape, generator=g, dtype=F32).to(dtype)


def _uniform(shape, lo, hi, g):
    return torch.empty(shape, dtype=F32).uniform_(lo, hi, generator=g)


def sdm_inputs(cfg: SdmConfig, T=None, seed=None):
    """Draw order: sw1, sw2, sr1, sr2, v, alpha, beta.  Shapes [B,T,H,*]."""
    T = cfg.T if T is None else T
    g = _gen(cfg.seed if seed is None else seed)
    B, H = cfg.B, cfg.H
    d = dict(
        sw1=_normal((B, T, H, cfg.sqrtN), g, cfg.dtype),
        sw2=_normal((B, T, H, cfg.sqrtN), g, cfg.dtype),
        sr1=_normal((B, T, H, cfg.sqrtN), g, cfg.dtype),
        sr2=_normal((B, T, H, cfg.sqrtN), g, cfg.dtype),
        v=_normal((B, T, H, cfg.d_v), g, cfg.dtype),
        alpha=_uniform((B, T, H), 0.9, 1.0, g),
        beta=_uniform((B, T, H), 0.0, 1.0, g),
    )
    return d


def gdn_inputs(cfg: GdnConfig, T=None, seed=None, B=None, H=None):
    """Draw order: q, k (normalised), v, beta, alpha.  Shapes [B,T,H,*]."""
    T = cfg.T if T is None else T
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    g = _gen(cfg.seed if seed is None else seed)
    q = _normal((B, T, H, cfg.d_k), g, cfg.dtype)
    kr = torch.randn((B, T, H, cfg.d_k), generator=g, dtype=F32)
    k = (kr / kr.norm(dim=-1, keepdim=True)).to(cfg.dtype)
    v = _normal((B, T, H, cfg.d_v), g, cfg.dtype)
    beta = torch.sigmoid(torch.randn((B, T, H), generator=g, dtype=F32))
    ashape = (B, T, H, cfg.d_k) if cfg.kda else (B, T, H)
    alpha = _uniform(ashape, 0.9, 1.0, g)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta)


def gdn2_inputs(cfg: GdnConfig, T=None, seed=None, B=None, H=None):
    """GDN2: the KDA draws (q, k, v, beta, alpha per channel), then the erase
    vector b = sigmoid(N(0,1)) per key channel and the write vector
    w = sigmoid(N(0,1)) per value column.  Shapes [B,T,H,*]; beta is unused."""
    x = gdn_inputs(cfg, T=T, seed=seed, B=B, H=H)
    T, B, H = x["q"].shape[1], x["q"].shape[0], x["q"].shape[2]
    g = _gen((cfg.seed if seed is None else seed) + 7919)
    x["erase"] = torch.sigmoid(torch.randn((B, T, H, cfg.d_k), generator=g, dtype=F32))
    x["write"] = torch.sigmoid(torch.randn((B, T, H, cfg.d_v), generator=g, dtype=F32))
    return x


def sse_inputs(cfg: SseConfig, T=None, seed=None, B=None, H=None):
    """Draw order: logits, q, k (softmax over c), v, lam.  Shapes [B,T,H,*]."""
    T = cfg.T if T is None else T
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    g = _gen(cfg.seed if seed is None else seed)
    logits = torch.randn((B, T, H, cfg.N), generator=g, dtype=F32)
    q = _normal((B, T, H, cfg.c), g, cfg.dtype)
    k = torch.softmax(torch.randn((B, T, H, cfg.c), generator=g, dtype=F32), dim=-1).to(cfg.dtype)
    v = _normal((B, T, H, cfg.d), g, cfg.dtype)
    lam = _uniform((B, T, H, cfg.c), 0.95, 1.0, g)
    return dict(logits=logits, q=q, k=k, v=v, lam=lam)


def to_numpy_f32(t):
    """Exact fp32 copy (bf16 values widen exactly) as a numpy array for the oracle."""
    return t.detach().to("cpu", F32).contiguous().numpy()
