"""Router inputs with exact score ties, built so that the tie rule alone
decides the selection (weekinpapers "BasisKV: Value Latents for
Communication and Key Routing", Abstract: the router chooses which Key pages
are read; the rule taken for equal scores is the larger score first, then
the smaller logical page, selections listed in ascending page order).

Two kinds of ties:

* summary ties: pages whose stored sums are the same bits and whose valid
  counts are equal get scores of the same bits on any implementation that
  computes a page's score from its own sums alone (the oracle in fp64, the
  GPU in fp32).  The sums are drawn here directly (no tokens), so only the
  router can use these cases.
* an appended page tying another page: the last page of a sequence is
  filled with a copy of an earlier full page's tokens, its last token written
  by the decode-step append.  Both pages then hold the same stored values, and
  each side computes both pages' sums the same way, so their scores tie.

Every case also checks that no other pair of scores lies within 1e-4
relative of the selection boundary, so that the oracle's fp32 scores and the
GPU's (which differ in the last bits) rank the untied pages alike.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

import oracle
from tests import cases
from workloads import synth
from workloads.configs import BF16, Workload

GAP = 1e-4  # relative separation required of distinct scores around the boundary


def order(scores: np.ndarray) -> List[int]:
    """Page indices by (score descending, index ascending)."""
    return sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))


def boundary_clean(scores: np.ndarray, k: int, tied: Sequence[int] = ()) -> bool:
    """True when the k-th and (k+1)-th ranked distinct scores are separated
    by more than GAP relative (pages in `tied` share one score and are
    exempt among themselves)."""
    o = order(scores)
    if k <= 0 or k >= len(o):
        return True
    vals = [float(scores[j]) for j in o]
    tied = set(tied)
    for i in range(max(0, k - 3), min(len(o) - 1, k + 2)):
        a, b = vals[i], vals[i + 1]
        if a == b and o[i] in tied and o[i + 1] in tied:
            continue
        if abs(a - b) <= GAP * max(abs(a), abs(b), 1e-30):
            return False
    return True


def summary_scenario(w: Workload, lengths: Sequence[int], seed: int):
    """A scenario whose cache holds only drawn page sums (the router's input)."""
    sc = cases.make_scenario(w, lengths=lengths, write=False)
    sc.cache = oracle.Cache(sc.d, sc.page_table)
    rng = np.random.default_rng(seed)
    RR = w.rank_v + w.rank_k
    for b, n in enumerate(sc.lengths):
        npg = -(-int(n) // w.page_size)
        for j in range(npg):
            cnt = min(w.page_size, int(n) - j * w.page_size)
            p = sc.page_table[b, j]
            # sums of `cnt` unit-variance values: std sqrt(cnt)
            sc.cache.summ[p] = (rng.standard_normal((w.n_kv_heads, RR)) * np.sqrt(cnt)).astype(np.float32)
    sc.W_ofT = oracle.fold(sc.d, sc.fac.B, sc.fac.W_O)
    return sc


def copy_sums(sc, b: int, src: int, dst: Sequence[int]) -> None:
    for j in dst:
        sc.cache.summ[sc.page_table[b, j]] = sc.cache.summ[sc.page_table[b, src]]


def straddle(sc, b: int, k: int, run: int = 5, ahead: int = 2) -> List[int]:
    """Give run - 1 low-ranked full pages the sums of the full page ranked
    k - ahead, some below it and some above it in page order: the tie run
    then occupies ranks k - ahead .. k - ahead + run - 1 and its `ahead`
    smallest pages are kept.  Returns the tied pages."""
    w = sc.w
    npg = int(sc.lengths[b]) // w.page_size  # full pages only: equal counts
    _, _, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    o = order(scores[b, 0, :npg])
    src = o[k - ahead]
    low = o[k + 8:]
    below = [j for j in low if j < src]
    above = [j for j in low if j > src]
    rng = np.random.default_rng(1000 + b)
    nb = min(len(below), (run - 1) // 2)
    dst = rng.choice(below, size=nb, replace=False).tolist() if nb else []
    dst += rng.choice(above, size=run - 1 - nb, replace=False).tolist()
    copy_sums(sc, b, src, dst)
    return sorted([src] + dst)


def append_tie_scenario(w: Workload, n: int, k: int, side: int, seed: int = 0):
    """One sequence of n tokens (n a multiple of the page size): its last page
    is made a copy of the full page that ranks k-1 (side 0: the pair ties at
    the last kept rank, the appended page loses) or k-2 (side 1: both are
    kept) among the other pages.  Returns the scenario (oracle cache holding
    every token) and the copied page."""
    assert n % w.page_size == 0
    ps = w.page_size
    w = w.with_(batch=1, top_k=k)
    sc = cases.make_scenario(w, lengths=[n], seed=seed)
    npg = n // ps
    _, _, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    o = order(scores[0, 0, :npg - 1])
    src = o[k - 1 - side]
    last = npg - 1
    sc.K[0][last * ps:n] = sc.K[0][src * ps:(src + 1) * ps]
    sc.V[0][last * ps:n] = sc.V[0][src * ps:(src + 1) * ps]
    sc.cache = oracle.Cache(sc.d, sc.page_table)
    oracle.write(sc.d, sc.fac, sc.cache, 0, 0, sc.K[0], sc.V[0])
    return sc, src


def expected(scores: np.ndarray, k: int) -> List[int]:
    """Top-k by the tie rule, ascending."""
    return sorted(order(scores)[:k])
