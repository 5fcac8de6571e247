"""The five benchmark/parity workloads, by shape.

C1  forward only, B1 H2 S128 D64, bidirectional T5 (32 buckets, max distance
    128), scale 1.0, no mask.
C2  encoder fwd+bwd, B16 H12 S1024 D64, bidirectional T5, scale 1.0.
C3  decoder fwd+bwd, B8 H12 S4096 D64, causal, unidirectional T5, scale 1.0.
C4  packed encoder fwd+bwd, 32768 tokens, lengths lognormal(6,1) clipped to
    [16,4096], H12 D64, bidirectional T5 within each sequence, scale 1.0.
C5  long-context causal fwd+bwd, B2 H16 S16384 D128, scale 1/sqrt(128), run
    once with ALiBi (slopes 2^(-8h/16)) and once with RoPE (base 10000).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    batch: int            # dense batch (1 for packed)
    seqlen: int           # dense sequence length (max length for packed)
    heads: int
    head_dim: int
    causal: bool
    bias: str             # "t5" | "alibi" | "none"
    bidirectional: bool
    scale: float
    rope_base: Optional[float] = None
    varlen_total: Optional[int] = None
    backward: bool = True
    num_buckets: int = 32
    max_distance: int = 128


CONFIGS = [
    Config("c1_fwd_b1h2s128d64_t5bi", 1, 1, 128, 2, 64, False, "t5", True, 1.0,
           backward=False),
    Config("c2_enc_b16h12s1024d64_t5bi", 2, 16, 1024, 12, 64, False, "t5", True, 1.0),
    Config("c3_dec_b8h12s4096d64_causal_t5uni", 3, 8, 4096, 12, 64, True, "t5", False, 1.0),
    Config("c4_varlen_t32768h12d64_t5bi", 4, 1, 4096, 12, 64, False, "t5", True, 1.0,
           varlen_total=32768),
    Config("c5a_long_b2h16s16384d128_causal_alibi", 5, 2, 16384, 16, 128, True, "alibi",
           False, 1.0 / math.sqrt(128.0)),
    Config("c5b_long_b2h16s16384d128_causal_rope", 5, 2, 16384, 16, 128, True, "none",
           False, 1.0 / math.sqrt(128.0), rope_base=10000.0),
]


def config_by_name(prefix: str) -> Config:
    for c in CONFIGS:
        if c.name.startswith(prefix):
            return c
    raise KeyError(prefix)
