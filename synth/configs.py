"""Workload shapes and input distributions.

Each entry restates one workload: the shapes, the weight format and the value
distributions of its synthetic inputs.  Nothing here computes any part of the
method.  The sizes follow the configurations the pages' engines run at: a
512-expert top-10 MoE layer with one always-on shared expert, a 288-expert
top-8 layer, 2,048-token prompt chunks and a 5120-wide dense model.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

FMT_E2M1 = 1        # 4-bit e2m1 codes, one fp8-e4m3 scale per 16 weights
FMT_E2M3 = 2        # 6-bit e2m3 codes, one power-of-two (UE8M0) scale per 128 weights
FMT_MXFP4 = 3       # 4-bit e2m1 codes, one UE8M0 scale per 32 weights
FMT_INT4_F16 = 4    # 4-bit two's-complement integers, one fp16 scale per 64 weights
FMT_E2M3_E4M3 = 5   # 6-bit e2m3 codes, one fp8-e4m3 scale per 16 weights
FORMATS = (FMT_E2M1, FMT_E2M3, FMT_MXFP4, FMT_INT4_F16, FMT_E2M3_E4M3)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    tokens: int
    hidden: int
    experts: int
    top_k: int
    inter: int
    shared_inter: int = 0            # 0: no shared expert
    fmt: int = FMT_E2M1
    logit_sigma: float = 1.0         # router logits ~ N(0, sigma), fp32
    x_sigma: float = 1.0             # hidden state ~ N(0, sigma), rounded to bf16
    scale_log2: Tuple[float, float] = (-6.0, -2.0)   # e4m3 scales: 2^U[lo, hi)
    ue8m0_exp: Tuple[int, int] = (-8, -3)           # UE8M0 scales: 2^e, e uniform integer
    fp16_log2: Tuple[float, float] = (-8.0, -4.0)   # fp16 scales (int4): 2^U[lo, hi)
    # the steps either side (the whole block): RMSNorm gains ~ 1 + N(0, gamma_sigma)
    # in bf16, its epsilon, and router weights ~ N(0, logit_sigma / sqrt(hidden))
    # in bf16, so that the scores of a unit-RMS activation have spread logit_sigma
    norm_eps: float = 1e-6
    gamma_sigma: float = 0.1
    seed: int = 0
    description: str = ""


@dataclass(frozen=True)
class GemvConfig:
    name: str
    rows: int
    cols: int
    batches: Tuple[int, ...]
    fmt: int = FMT_E2M3
    ue8m0_exp: Tuple[int, int] = (-8, -3)
    scale_log2: Tuple[float, float] = (-6.0, -2.0)
    fp16_log2: Tuple[float, float] = (-8.0, -4.0)
    x_sigma: float = 1.0
    seed: int = 0
    description: str = ""


TOY = MoEConfig("toy_decode", tokens=1, hidden=256, experts=8, top_k=2, inter=512,
                description="toy MoE decode layer: 1 token, H=256, 8 experts, top-2, I=512")
GEMV = GemvConfig("dense_gemv_e2m3", rows=25600, cols=5120, batches=(1, 4),
                  description="dense block-scaled GEMV: W 25600x5120 e2m3 + UE8M0/128, x bf16, B=1 and 4")
WIDE = MoEConfig("wide_decode", tokens=1, hidden=2048, experts=512, top_k=10, inter=512,
                 shared_inter=512, logit_sigma=1.5,
                 description="wide MoE decode layer: 1 token, H=2048, 512 experts + 1 shared, top-10, I=512")
BATCHED = MoEConfig("batched_decode", tokens=16, hidden=6144, experts=288, top_k=8, inter=2048,
                    description="batched-decode MoE layer: 16 tokens, H=6144, 288 experts, top-8, I=2048")
PREFILL = MoEConfig("prefill", tokens=2048, hidden=2048, experts=512, top_k=10, inter=512,
                    description="prefill MoE layer: 2048 tokens, H=2048, 512 experts, top-10, I=512")

# The wide decode layer with the steps either side: RMSNorm, router scores and
# top-k, the MoE layer, the residual add.
WIDE_BLOCK = MoEConfig("wide_block", tokens=1, hidden=2048, experts=512, top_k=10, inter=512, shared_inter=512,
                       logit_sigma=1.5,
                       description="wide MoE block: RMSNorm, router GEMV + top-10 of 512, the layer, residual add")
BATCHED_BLOCK = MoEConfig("batched_block", tokens=16, hidden=6144, experts=288, top_k=8, inter=2048,
                          description="batched MoE block: RMSNorm, router GEMV + top-8 of 288, the layer, residual add")

ALL = {c.name: c for c in (TOY, GEMV, WIDE, BATCHED, PREFILL, WIDE_BLOCK, BATCHED_BLOCK)}
