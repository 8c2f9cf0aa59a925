"""The five workloads of the hybrid-attention hot path, as frozen dataclasses.

Sizes follow the hybrid long-context attention described on the group-reading
wiki page "DeepSeek-V4 深度研究剖析" §5.2-§5.4: a sliding window of 128 raw
tokens, CSA with 4:1 compression and a per-query top-k (512 for Flash, 1024 for
Pro), HCA with 128:1 compression attended densely, all over one shared KV head
(page 1, "Deep dive" §14).  The shapes of each workload (batch, context, heads,
precision) are the workload definitions of this library's benchmark suite.

This module holds no arithmetic of the method: only names and sizes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "decode" | "ragged"
    seed: int
    H: int                    # query heads (one shared KV head)
    d: int = 128              # head dim of Q/K/V
    n_win: int = 128          # SWA window (raw tokens, the query included)
    m_csa: int = 4            # CSA compression ratio
    k_csa: int = 512          # CSA per-query top-k
    m_hca: int = 128          # HCA compression ratio
    H_I: int = 4              # indexer heads
    d_I: int = 64             # indexer head dim
    layers: Tuple[str, ...] = ("csa", "hca")
    kv_dtype: str = "bf16"    # storage of compressed K/V: "bf16" | "fp8"
    T: int = 0                # prefill: sequence length
    B: int = 0                # decode: batch
    L: int = 0                # decode: cached tokens per request (new token at t = L)
    planted: bool = False     # prefill 128K: correlated keys every 4096 tokens
    paged_shuffle: bool = False
    steps: int = 0            # ragged: decode steps
    L_min: int = 0            # ragged: log-uniform context range
    L_max: int = 0
    page_size: int = 64
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    def m(self, layer: str) -> int:
        return self.m_csa if layer == "csa" else self.m_hca


PREFILL_4K = Workload(
    name="prefill_4k", kind="prefill", seed=1001, H=16, T=4096, k_csa=64,
    layers=("csa", "hca"))

CSA_DECODE_128K = Workload(
    name="csa_decode_128k", kind="decode", seed=1002, H=64, B=32, L=131072,
    k_csa=512, layers=("csa",))

HYBRID_PREFILL_128K = Workload(
    name="hybrid_prefill_128k", kind="prefill", seed=1003, H=64, T=131072,
    k_csa=512, layers=("csa", "hca"), planted=True)

PRO_DECODE_1M = Workload(
    name="pro_decode_1m", kind="decode", seed=1004, H=128, B=4, L=1048576,
    k_csa=1024, layers=("csa", "hca"), kv_dtype="fp8")

RAGGED_SERVING = Workload(
    name="ragged_serving", kind="ragged", seed=1005, H=64, B=16, k_csa=1024,
    layers=("csa", "hca"), paged_shuffle=True, steps=256,
    L_min=8192, L_max=1048576)

ALL = (PREFILL_4K, CSA_DECODE_128K, HYBRID_PREFILL_128K, PRO_DECODE_1M,
       RAGGED_SERVING)
BY_NAME = {w.name: w for w in ALL}


def shrink(w: Workload, **kw) -> Workload:
    """A smaller variant of a workload (same structure, smaller sizes)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)
