"""The exact-tie router cases shared by the CPU check of their construction
(tests/test_tie_cases.py) and the GPU comparison (tests/test_gpu_ties.py).

Each builder returns (scenario, top_k, tied pages per row, description).
The shapes take the router down both of its selection paths: at most 512
pages with 2 <= top_k <= 64, and the wider selections (top_k above 64, or
more than 512 pages).
"""
from __future__ import annotations

from tests import tie_cases as tc
from workloads import configs

BASE = configs.get("llama8b_32k")

# (name, pages per row, top_k)
SUMMARY_SHAPES = [
    ("net_k40_p300", 300, 40),     # sorting-network path
    ("radix_k100_p300", 300, 100),  # top_k above 64
    ("radix_k40_p700", 700, 40),    # more than 512 pages
    ("k1_p64", 64, 1),              # a single page
]


def summary_case(name: str):
    """Three rows: a tie run straddling the boundary (two of five kept), every
    page tied (all scores equal: the first top_k pages are kept), and a tie
    run entirely inside the kept set followed by a clean boundary."""
    shape = dict((s[0], s[1:]) for s in SUMMARY_SHAPES)[name]
    npg, k = shape
    ps = BASE.page_size
    w = BASE.with_(name=f"tie_{name}", cfg_id=300 + npg + k, batch=3, top_k=k, d_model=256, ctx=npg * ps)
    for seed in range(20):
        sc = tc.summary_scenario(w, [npg * ps] * 3, seed)
        tied = [[], [], []]
        if k >= 2:
            tied[0] = tc.straddle(sc, 0, k, run=5, ahead=2)
        else:  # top_k 1: three pages share the best score, the smallest is kept
            tied[0] = tc.straddle(sc, 0, 1, run=3, ahead=1)
        tc.copy_sums(sc, 1, 0, range(1, npg))
        tied[1] = list(range(npg))
        if k >= 4:
            tied[2] = tc.straddle(sc, 2, k, run=3, ahead=k // 2)  # run well inside the kept set
        import oracle
        _, _, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
        if all(tc.boundary_clean(scores[b, 0, :npg], k, tied[b]) for b in (0, 2)):
            return sc, k, tied
    raise AssertionError(f"no seed gives a clean boundary for {name}")


# (name, pages, top_k, side): side 0 = the appended page ties the last kept
# page and loses the tie; side 1 = it ties the next-to-last kept page and
# both are kept
APPEND_SHAPES = [
    ("net_side0", 200, 40, 0),
    ("net_side1", 200, 40, 1),
    ("radix_side0", 200, 80, 0),
    ("radix_side1", 200, 80, 1),
]


def append_case(name: str):
    npg, k, side = dict((s[0], s[1:]) for s in APPEND_SHAPES)[name]
    ps = BASE.page_size
    import oracle
    for seed in range(20):
        w = BASE.with_(name=f"atie_{name}", cfg_id=400 + k, d_model=256, ctx=npg * ps)
        sc, src = tc.append_tie_scenario(w, npg * ps, k, side, seed=seed)
        _, _, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
        if tc.boundary_clean(scores[0, 0, :npg], k, [src, npg - 1]):
            return sc, k, src, side
    raise AssertionError(f"no seed gives a clean boundary for {name}")
