"""Workload shapes for the routed latent decode path.

Each workload is one GPU's tensor-parallel share of an attention layer: its
query heads, the KV heads they share (grouped-query attention, Baidu article
"KV cache compression architectures", section on GQA) and its slice of the
output projection.  The cache is paged (machinelearning.ru "KV-кэширование",
section on storage formats); Values are kept only as rank-r latents and a
Key-specific residual of rank r_k is kept for routing (weekinpapers
"BasisKV: Value Latents for Communication and Key Routing", Abstract).

The five shapes are the decode and prefill workloads this library is sized
for:

* ``tiny_f32``     - 1 sequence, 1 query head on 1 KV head, head_dim 64,
                     1024 tokens in 64 pages of 16, r=16, r_k=8, top-k 8,
                     d_model 256, fp32 storage.  Small enough for the CPU
                     oracle to run everything.
* ``llama8b_32k``  - Llama-3-8B tensor-parallel-8 share: batch 16, 4 query
                     heads on 1 KV head, head_dim 128, 32768 tokens in pages
                     of 64, r=32, r_k=16, top-k 64, d_model 4096, bf16.
* ``llama70b_128k``- Llama-3-70B tensor-parallel-8 share: batch 32, 8 query
                     heads on 1 KV head, 131072 tokens, top-k 128,
                     d_model 8192, bf16.
* ``prefill_8k``   - one 8192-token prompt written and attended causally in
                     chunks of 2048, 8 query heads on 2 KV heads, r=48,
                     r_k=16, top-k = all pages, d_model 4096, bf16.
* ``ragged_mix``   - 64 sequences with lengths uniform in [1024, 65536],
                     pages scattered by a random permutation, 4 query heads
                     on 1 KV head, top-k = min(64, pages), d_model 4096, bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple

F32 = 0
BF16 = 1
DTYPE_NAMES = {F32: "f32", BF16: "bf16"}
DTYPE_BYTES = {F32: 4, BF16: 2}


@dataclass(frozen=True)
class Workload:
    """One GPU's share of one attention layer plus the cache geometry."""

    name: str
    cfg_id: int                 # seeds are keyed by this id
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    rank_v: int
    rank_k: int
    top_k: int
    d_model: int
    dtype: int                  # F32 or BF16
    ctx: int                    # tokens per sequence after the decode append (fixed-length workloads)
    length_range: Optional[Tuple[int, int]] = None   # ragged: inclusive uniform range
    permuted_pages: bool = False
    prefill_chunk: Optional[int] = None               # prefill workloads: queries per chunk
    sink_pages: int = 0         # routing: first pages always kept (0: plain top-k)
    local_pages: int = 0        # routing: last pages always kept
    group_mean: int = 0         # routing: group score = mean over its query heads (0: max)
    head_select: int = 0        # routing: every query head selects its own pages (0: per KV head)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def units(self) -> int:
        """Selection units per sequence: KV heads, or query heads with head_select."""
        return self.n_q_heads if self.head_select else self.n_kv_heads

    @property
    def max_ctx(self) -> int:
        return self.length_range[1] if self.length_range else self.ctx

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.max_ctx // self.page_size)

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", cfg_id=0, batch=1, n_q_heads=1, n_kv_heads=1,
        head_dim=64, page_size=16, rank_v=16, rank_k=8, top_k=8,
        d_model=256, dtype=F32, ctx=1024),
    "llama8b_32k": Workload(
        name="llama8b_32k", cfg_id=1, batch=16, n_q_heads=4, n_kv_heads=1,
        head_dim=128, page_size=64, rank_v=32, rank_k=16, top_k=64,
        d_model=4096, dtype=BF16, ctx=32768),
    "llama70b_128k": Workload(
        name="llama70b_128k", cfg_id=2, batch=32, n_q_heads=8, n_kv_heads=1,
        head_dim=128, page_size=64, rank_v=32, rank_k=16, top_k=128,
        d_model=8192, dtype=BF16, ctx=131072),
    "prefill_8k": Workload(
        name="prefill_8k", cfg_id=3, batch=1, n_q_heads=8, n_kv_heads=2,
        head_dim=128, page_size=64, rank_v=48, rank_k=16, top_k=128,
        d_model=4096, dtype=BF16, ctx=8192, prefill_chunk=2048),
    "ragged_mix": Workload(
        name="ragged_mix", cfg_id=4, batch=64, n_q_heads=4, n_kv_heads=1,
        head_dim=128, page_size=64, rank_v=32, rank_k=16, top_k=64,
        d_model=4096, dtype=BF16, ctx=0, length_range=(1024, 65536),
        permuted_pages=True),
}

BY_ID = {w.cfg_id: w for w in WORKLOADS.values()}


def get(name_or_id) -> Workload:
    if isinstance(name_or_id, int):
        return BY_ID[name_or_id]
    return WORKLOADS[name_or_id]
