"""Algorithmic byte and flop counts for one decode layer step and one prefill.

"Algorithmic" means what the method must move, counted once: the page sums of
every valid page (routing reads them all), the exact Keys and the latents of
the valid tokens of the selected pages, the page-table entries, the queries,
the new token's write, the folded output projection, the output and the
factors.  Split-K partials, re-reads and LDS traffic are not counted.

The KV-size formula 2 * L * H * d_h * n * bytes (Baidu article "KV cache
compression architectures", section 4; machinelearning.ru "KV-кэширование",
"Математическая формализация") is ``dense_kv_bytes``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np

from .configs import Workload


def dense_kv_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int, elem_bytes: int) -> int:
    """Bytes of a dense K+V cache."""
    return 2 * layers * kv_heads * head_dim * tokens * elem_bytes


@dataclass
class StepBytes:
    summaries: int
    keys: int
    latents: int
    page_table: int
    queries: int
    append: int
    w_of: int
    out: int
    factors: int

    @property
    def total(self) -> int:
        return (self.summaries + self.keys + self.latents + self.page_table + self.queries
                + self.append + self.w_of + self.out + self.factors)

    @property
    def attend_kernel(self) -> int:
        """Bytes of the gathered exact-QK attention alone (its per-launch unit)."""
        return self.keys + self.latents + self.queries + self.attend_meta

    attend_meta: int = 0


def _valid_selected_tokens(n: int, ps: int, k_eff: int, sel: Optional[np.ndarray]) -> int:
    npg = -(-n // ps)
    if sel is None:
        # top-k over a full context: every selected page is full unless the last
        # page is selected; count the worst case (all full) capped by n.
        return min(k_eff * ps, n)
    tot = 0
    for j in sel[:k_eff]:
        tot += min(ps, n - int(j) * ps)
    return tot


def decode_step_bytes(w: Workload, lengths: Sequence[int],
                      selections: Optional[np.ndarray] = None,
                      n_selected: Optional[np.ndarray] = None) -> StepBytes:
    """Algorithmic bytes of one decode layer step (append, route, attend, project).

    ``selections`` [B][U][top_k] (U selection units per row, w.units) gives exact valid-token counts
    for partially filled selected pages; without it every selected page is
    counted full (capped by the sequence length).
    """
    eb, ps, D, R, RK = w.elem_bytes, w.page_size, w.head_dim, w.rank_v, w.rank_k
    G = w.group
    GU = 1 if w.head_select else G   # query heads per selection unit
    s = dict(summaries=0, keys=0, latents=0, page_table=0, queries=0, append=0)
    meta = 0
    for b, n in enumerate(lengths):
        n = int(n)
        npg = -(-n // ps)
        for g in range(w.n_kv_heads):
            s["summaries"] += npg * (R + RK) * 4
            s["page_table"] += npg * 4
            s["queries"] += G * D * eb
            # new token: k and v in; K, latent and residual out; page sums read+written
            s["append"] += 2 * D * eb + (D + R + RK) * eb + 2 * (R + RK) * 4
        # each selection unit (a KV head, or a query head with head_select)
        # reads the Keys and latents of its own pages
        for u in range(w.units):
            k_eff = min(w.top_k, npg)
            sel = None if selections is None else selections[b, u]
            if n_selected is not None:
                k_eff = int(n_selected[b, u])
            tok = _valid_selected_tokens(n, ps, k_eff, sel)
            s["keys"] += tok * D * eb
            s["latents"] += tok * R * eb
            meta += 2 * k_eff * 4 + GU * R * 4   # selection ids, their page-table entries, z-hat out
    w_of = w.n_q_heads * R * w.d_model * eb
    out = len(lengths) * w.d_model * 4
    factors = w.n_kv_heads * (2 * D * R + 2 * D * RK) * 4
    sb = StepBytes(w_of=w_of, out=out, factors=factors, **s)
    sb.attend_meta = meta
    return sb


def decode_step_flops(w: Workload, lengths: Sequence[int]) -> Dict[str, int]:
    """Multiply-add flops (2 per MAC) of one decode step, full selected pages."""
    D, R, RK, ps, G = w.head_dim, w.rank_v, w.rank_k, w.page_size, w.group
    route = attend = append = 0
    for n in lengths:
        npg = -(-int(n) // ps)
        k_eff = min(w.top_k, npg)
        tok = min(k_eff * ps, int(n))
        for _ in range(w.n_kv_heads):
            append += 2 * (D * R + R * D + D * RK)
            route += 2 * G * (R + RK) * D + 2 * G * npg * (R + RK)
            attend += 2 * G * tok * (D + R)
    project = 2 * len(lengths) * w.n_q_heads * R * w.d_model
    return dict(append=append, route=route, attend=attend, project=project,
                total=append + route + attend + project)


def prefill_flops(w: Workload, start: int, n_tok: int) -> Dict[str, int]:
    """Flops of one causal prefill chunk of queries [start, start+n_tok)."""
    D, R, RK = w.head_dim, w.rank_v, w.rank_k
    keys = sum(p + 1 for p in range(start, start + n_tok))   # causal key count
    attn = 2 * w.n_q_heads * keys * (D + R)
    write = 2 * n_tok * w.n_kv_heads * (D * R + R * D + D * RK)
    proj = 2 * n_tok * w.n_q_heads * R * w.d_model
    return dict(attention=attn, writer=write, projection=proj, total=attn + write + proj)
