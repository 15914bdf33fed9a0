"""CPU check of the exact-tie router cases: the constructions produce the
tie structure they claim (tied pages share the same fp32 score bits, the
boundary is clean elsewhere) and the oracle keeps the pages the tie rule
names (weekinpapers "BasisKV: Value Latents for Communication and Key
Routing", Abstract: choosing which Key pages to read; equal scores go to the
smaller page)."""
import numpy as np
import pytest

import oracle
from tests import tie_cases as tc
from tests import tie_constructions as tk


@pytest.mark.parametrize("name", [s[0] for s in tk.SUMMARY_SHAPES])
def test_summary_tie_construction(name):
    sc, k, tied = tk.summary_case(name)
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    npg = int(sc.lengths[0]) // sc.w.page_size
    for b in range(sc.batch):
        s = scores[b, 0, :npg]
        t = tied[b]
        assert len({s[j].tobytes() for j in t}) <= 1, "tied pages must share their score bits"
        want = tc.expected(s, k)
        assert sel[b, 0, :k].tolist() == want
        assert int(n_sel[b, 0]) == k
        assert (sel[b, 0, k:] == -1).all()
    # row 0: exactly `ahead` of the run kept, the smallest of its pages
    s0 = sel[0, 0, :k].tolist()
    kept = [j for j in tied[0] if j in s0]
    ahead = 2 if k >= 2 else 1
    assert kept == sorted(tied[0])[:ahead]
    # row 1: every score equal -> the first k pages
    assert sel[1, 0, :k].tolist() == list(range(k))
    # row 2: the whole run kept
    if tied[2]:
        assert set(tied[2]) <= set(sel[2, 0, :k].tolist())


@pytest.mark.parametrize("name", [s[0] for s in tk.APPEND_SHAPES])
def test_append_tie_construction(name):
    sc, k, src, side = tk.append_case(name)
    npg = int(sc.lengths[0]) // sc.w.page_size
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    s = scores[0, 0, :npg]
    assert s[src] == s[npg - 1]
    chosen = sel[0, 0, :k].tolist()
    assert chosen == tc.expected(s, k)
    assert src in chosen
    assert (npg - 1 in chosen) == (side == 1)
