"""The five MSA forward workloads this library is measured and checked on.

Each is a synthetic stand-in for the pages' unpublished internal workloads
(a 109B-parameter model, 1M-token context; talk summary "How MiniMax M3 Was
Built", section on the index branch, and the "MiniMax稀疏注意力" topic page's
summary).  Every tensor is bf16 and i.i.d. N(0, 1) from a seed; the two
mid-size prefill workloads add a per-64-token-block N(0, 0.5) offset to the
keys so that block scores are not near-tied.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_q: int           # query rows per sequence (1 for decode)
    seq_kv: int          # key/value capacity per sequence (tokens)
    q_start: int         # position of query row 0 (prefill / chunked prefill)
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_idx_heads: int
    idx_head_dim: int
    block_size: int
    top_k: int
    decode: bool
    block_offset_std: float  # std of the per-block key offset (0 = none)
    fused_topk: bool         # block scores must stream through a running top-k
    seed: int
    iq_shared_rows: int = 1  # rows per run that share one index query (1 = independent)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def nblk(self) -> int:
        return (self.seq_kv + self.block_size - 1) // self.block_size

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def shrink(self, **kw) -> "Workload":
        return replace(self, **kw)


_COMMON = dict(head_dim=128, n_idx_heads=4, idx_head_dim=64, block_size=64)

TINY_PREFILL_2K = Workload("tiny_prefill_2k", batch=1, seq_q=2048, seq_kv=2048, q_start=0,
                           n_q_heads=8, n_kv_heads=2, top_k=8, decode=False,
                           block_offset_std=0.0, fused_topk=False, seed=20260001, **_COMMON)
PREFILL_32K = Workload("prefill_32k", batch=1, seq_q=32768, seq_kv=32768, q_start=0,
                       n_q_heads=32, n_kv_heads=4, top_k=32, decode=False,
                       block_offset_std=0.5, fused_topk=False, seed=20260002, **_COMMON)
PREFILL_128K = Workload("prefill_128k", batch=1, seq_q=131072, seq_kv=131072, q_start=0,
                        n_q_heads=32, n_kv_heads=4, top_k=64, decode=False,
                        block_offset_std=0.5, fused_topk=False, seed=20260003, **_COMMON)
DECODE_32x256K = Workload("decode_32x256k", batch=32, seq_q=1, seq_kv=262144, q_start=0,
                          n_q_heads=32, n_kv_heads=4, top_k=64, decode=True,
                          block_offset_std=0.0, fused_topk=False, seed=20260004, **_COMMON)
CHUNK_1M = Workload("chunk_prefill_1m", batch=1, seq_q=8192, seq_kv=1048576, q_start=1040384,
                    n_q_heads=32, n_kv_heads=4, top_k=128, decode=False,
                    block_offset_std=0.0, fused_topk=True, seed=20260005, **_COMMON)

ALL = [TINY_PREFILL_2K, PREFILL_32K, PREFILL_128K, DECODE_32x256K, CHUNK_1M]

# Diagnostic workloads (not among the five above): every 64-row query block
# shares one index query, so its rows select the same blocks.  Real index
# queries of neighbouring tokens are correlated to some degree; these show the
# sparse prefill where a tile's rows agree, the regime opposite to the
# independent draws above.
PREFILL_128K_SHARED_IQ = PREFILL_128K.shrink(name="prefill_128k_shared_iq", iq_shared_rows=64)
PREFILL_32K_SHARED_IQ = PREFILL_32K.shrink(name="prefill_32k_shared_iq", iq_shared_rows=64)
DIAGNOSTIC = [PREFILL_32K_SHARED_IQ, PREFILL_128K_SHARED_IQ]

BY_NAME = {w.name: w for w in ALL + DIAGNOSTIC}
