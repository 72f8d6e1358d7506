"""Workload shapes for the P-EAGLE parallel-draft step.

Each workload fixes the drafter shape, the draft depth K, the batch and how the
synthetic inputs are drawn.  The shapes follow the 20B-class drafter described
on "P-EAGLE: parallel speculative decoding in vLLM" (Architecture and
mechanism: an N-layer Transformer plus LM head over concat(emb, h) inputs) and
the sequence-length statistics quoted on "AWS and vLLM ship P-EAGLE" (How it
works: prompt+generation median 3891, p90 10800 tokens).  Nothing here
computes any part of the method.
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # 1-based; the seed is 1000 + index
    batch: int                 # B, requests
    K: int                     # draft depth (num_speculative_tokens)
    d: int                     # hidden size
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    mlp: int                   # I
    layers: int                # L
    vocab: int                 # V
    dtype: str                 # "f32" or "bf16"
    prefix: Tuple[str, float, float] = ("fixed", 64, 0)   # p0 distribution
    accepted: str = "uniform"  # "uniform" over 0..K, or an int as text
    weight_std: float = 0.02   # N(0, std) for linear and embedding weights
    block_size: int = 16
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    Ks: Tuple[int, ...] = field(default=())   # K sweep (workload 4)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def slots(self) -> int:
        return 2 * self.K

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload("tiny_f32", 1, batch=1, K=4, d=256, n_q_heads=4, n_kv_heads=2,
                head_dim=64, mlp=1024, layers=1, vocab=1024, dtype="f32",
                prefix=("fixed", 64, 0), accepted="2", weight_std=1.0 / 16.0)

C1 = Workload("c1_20b", 2, batch=1, K=7, d=2880, n_q_heads=64, n_kv_heads=8,
              head_dim=64, mlp=7680, layers=1, vocab=201088, dtype="bf16",
              prefix=("fixed", 2048, 0))

# lognormal: median 3891, sigma from p90 = 10800 = 3891 * exp(1.2816 sigma)
C64 = Workload("c64_20b", 3, batch=64, K=7, d=2880, n_q_heads=64, n_kv_heads=8,
               head_dim=64, mlp=7680, layers=1, vocab=201088, dtype="bf16",
               prefix=("lognormal", 3891.0, 0.7966))

KSWEEP = Workload("ksweep_2b", 4, batch=16, K=7, d=2048, n_q_heads=32, n_kv_heads=4,
                  head_dim=64, mlp=6144, layers=4, vocab=151936, dtype="bf16",
                  prefix=("fixed", 4096, 0), Ks=(1, 3, 5, 7, 11, 15))

MAXB = Workload("maxbatch_20b", 5, batch=256, K=7, d=2880, n_q_heads=64, n_kv_heads=8,
                head_dim=64, mlp=7680, layers=1, vocab=201088, dtype="bf16",
                prefix=("uniform", 256, 8192))

ALL = (TINY, C1, C64, KSWEEP, MAXB)
BY_NAME = {w.name: w for w in ALL}
