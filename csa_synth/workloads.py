"""The five workloads the CSA / HCA path is built and measured on.

Shapes follow the parameters the technical review gives for V4-Pro
("DeepSeek V4 技术解读", §2.1 CSA: m = 4, 64 indexer heads of dim 128,
top-k = 1024; §2.2 HCA: m' = 128) and the 128K - 1M token contexts the
pages discuss (§2.4, one-million-token context).  Values the pages leave
open (batch sizes, core head count, distributions, seeds) are readings,
recorded here once so every consumer sees the same numbers.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str               # "csa" or "hca"
    B: int                  # sequences
    m: int                  # tokens pooled per compressed entry
    n_cache: int            # entries already in the cache (drawn directly)
    n_raw: int              # raw tokens pooled by the compress stage (appended after the cache)
    Tq: int                 # query tokens per sequence
    q_pos0: int             # position of the first query token
    H: int                  # core-attention query heads (one shared KV head)
    D: int                  # core-attention head dim
    H_I: int                # indexer heads (0 for HCA)
    D_I: int                # indexer head dim (0 for HCA)
    k: int                  # top-k entries per query (0 for HCA: all visible)
    dtype: str              # storage dtype of q / caches / raw tokens: "f32" | "bf16"
    index_dtype: str        # indexer q/k storage: "f32" | "bf16" | "fp4" | "mx4"
    w_std: float            # std of the indexer head weights
    seed: int

    @property
    def N(self) -> int:
        """Cache rows per sequence after the compress stage."""
        return self.n_cache + self.n_raw // self.m

    @property
    def C(self) -> int:
        """Channels per raw token that the compress stage pools: K | V | K_I."""
        return 2 * self.D + (self.D_I if self.kind == "csa" else 0)

    def visible(self, t: int) -> int:
        """Entries visible to query position t (entry j visible iff m(j+1) <= t+1)."""
        return min(self.N, (t + 1) // self.m)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 case: 256 raw tokens, every position queries.
    "tiny_csa": Workload(
        name="tiny_csa", kind="csa", B=1, m=4, n_cache=0, n_raw=256, Tq=256, q_pos0=0,
        H=4, D=64, H_I=4, D_I=32, k=16, dtype="f32", index_dtype="f32",
        w_std=1.0 / 2.0, seed=0),
    # CSA decode, 128K context: the headline workload.
    "csa_decode_128k": Workload(
        name="csa_decode_128k", kind="csa", B=16, m=4, n_cache=32768, n_raw=0, Tq=1,
        q_pos0=131072, H=64, D=128, H_I=64, D_I=128, k=1024, dtype="bf16",
        index_dtype="bf16", w_std=1.0 / 8.0, seed=1),
    # CSA prefill chunk: 4096 new tokens after a 262144-token context.
    "csa_prefill_chunk": Workload(
        name="csa_prefill_chunk", kind="csa", B=1, m=4, n_cache=65536, n_raw=4096, Tq=4096,
        q_pos0=262144, H=64, D=128, H_I=64, D_I=128, k=1024, dtype="bf16",
        index_dtype="bf16", w_std=1.0 / 8.0, seed=2),
    # HCA decode at 1M context: 1048576 raw tokens pooled 128:1.
    "hca_decode_1m": Workload(
        name="hca_decode_1m", kind="hca", B=32, m=128, n_cache=0, n_raw=1048576, Tq=1,
        q_pos0=1048576, H=64, D=128, H_I=0, D_I=0, k=0, dtype="bf16",
        index_dtype="bf16", w_std=0.0, seed=3),
    # CSA decode at 1M context with an FP4 E2M1 indexer.
    "csa_decode_1m_fp4": Workload(
        name="csa_decode_1m_fp4", kind="csa", B=4, m=4, n_cache=262144, n_raw=0, Tq=1,
        q_pos0=1048576, H=64, D=128, H_I=64, D_I=128, k=1024, dtype="bf16",
        index_dtype="fp4", w_std=1.0 / 8.0, seed=4),
    # The same with power-of-two (E8M0) block scales, the MX FP4 encoding that
    # gfx950's block-scaled MFMA applies itself (same draws as the fp4 case).
    "csa_decode_1m_mx4": Workload(
        name="csa_decode_1m_mx4", kind="csa", B=4, m=4, n_cache=262144, n_raw=0, Tq=1,
        q_pos0=1048576, H=64, D=128, H_I=64, D_I=128, k=1024, dtype="bf16",
        index_dtype="mx4", w_std=1.0 / 8.0, seed=4),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def std_for_dim(dim: int) -> float:
    """Q / K / V / indexer vectors are drawn N(0, 1) / sqrt(dim)."""
    return 1.0 / math.sqrt(dim)
