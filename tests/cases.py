"""Shared test scaffolding: seeded scenarios built on the CPU oracle.

A scenario is a workload shape, its seeded factors, sequence lengths, page
table, per-sequence Keys/Values and queries, and (optionally) the oracle's
cache with every token written.  GPU tests upload the same host arrays.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

import oracle
from workloads import synth
from workloads.configs import BF16, F32, Workload


def small(name: str, cfg_id: int, **kw) -> Workload:
    base = dict(name=name, cfg_id=cfg_id, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=16,
                page_size=4, rank_v=4, rank_k=2, top_k=3, d_model=24, dtype=F32, ctx=37)
    base.update(kw)
    return Workload(**base)


@dataclass
class Scenario:
    w: Workload
    fac: synth.Factors
    rows: List[int]                 # global sequence ids (generator keys) of the local rows
    lengths: np.ndarray             # tokens per local row after the decode append
    page_table: np.ndarray
    num_pages: int
    K: List[np.ndarray] = field(default_factory=list)   # per row [n][H_kv][d_h] storage dtype
    V: List[np.ndarray] = field(default_factory=list)
    q: Optional[np.ndarray] = None  # [rows][H_q][d_h]
    d: Optional[oracle.Dims] = None
    cache: Optional[oracle.Cache] = None
    W_ofT: Optional[np.ndarray] = None

    @property
    def batch(self) -> int:
        return len(self.rows)


def make_scenario(w: Workload, seed: int = 0, rows: Optional[Sequence[int]] = None,
                  lengths: Optional[Sequence[int]] = None, permuted: Optional[bool] = None,
                  write: bool = True, upto_last: bool = False, fill=0) -> Scenario:
    """Build inputs for `rows` (default: the whole batch).

    With ``write`` the oracle cache holds every token (or all but the last when
    ``upto_last``: the decode step then appends the last one).
    """
    fac = synth.make_factors(w, seed)
    all_len = synth.make_lengths(w, seed)
    rows = list(range(w.batch)) if rows is None else list(rows)
    if lengths is None:
        lengths = [int(all_len[r]) for r in rows]
    lengths = np.asarray(lengths, np.int32)
    pt, total = synth.make_page_table(w, lengths, seed, permuted)
    sc = Scenario(w=w, fac=fac, rows=rows, lengths=lengths, page_table=pt, num_pages=total)
    for r, n in zip(rows, lengths):
        Kf, Vf = synth.make_sequence(w, fac, r, max(int(n), 1), seed)
        sc.K.append(Kf[:n])
        sc.V.append(Vf[:n])
    qall = synth.make_queries(w, seed=seed)
    sc.q = np.ascontiguousarray(qall[rows])
    sc.d = oracle.Dims.of(w, batch=len(rows), num_pages=total)
    if write:
        sc.cache = oracle.Cache(sc.d, pt, fill)
        for b, n in enumerate(lengths):
            m = int(n) - 1 if upto_last else int(n)
            if m > 0:
                oracle.write(sc.d, fac, sc.cache, b, 0, sc.K[b][:m], sc.V[b][:m])
        sc.W_ofT = oracle.fold(sc.d, fac.B, fac.W_O)
    return sc


def all_pages_selection(lengths: Sequence[int], n_kv: int, top_k: int, ps: int):
    B = len(lengths)
    sel = np.full((B, n_kv, top_k), -1, np.int32)
    n_sel = np.zeros((B, n_kv), np.int32)
    for b, n in enumerate(lengths):
        npg = -(-int(n) // ps)
        assert npg <= top_k
        sel[b, :, :npg] = np.arange(npg)
        n_sel[b, :] = npg
    return sel, n_sel


def to_f64(x: np.ndarray, dtype: int) -> np.ndarray:
    return synth.storage_to_f64(x, dtype)


def softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s)
    e = np.exp(s - m)
    return e / e.sum()


def brute_topk(scores: np.ndarray, k: int) -> List[int]:
    """Indices of the k best scores, ties to the smaller index, ascending."""
    order = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    return sorted(order[:k])


def check_selection_valid(ref_scores: np.ndarray, chosen: Sequence[int], k: int, rtol: float):
    """`chosen` is a top-k of ref_scores up to swaps of near-equal scores."""
    chosen = list(chosen)
    assert len(chosen) == k == len(set(chosen))
    assert chosen == sorted(chosen)
    if k == len(ref_scores) or k == 0:
        return
    rest = [j for j in range(len(ref_scores)) if j not in set(chosen)]
    lo = min(float(ref_scores[j]) for j in chosen)
    hi = max(float(ref_scores[j]) for j in rest)
    assert lo >= hi - rtol * max(abs(lo), abs(hi), 1e-30), (lo, hi)


def check_outputs_on_selection(sc, sel, n_sel, z, out):
    """GPU outputs against the oracle's decode over the GPU's own selection
    (the reading for several correct selections: the sets may differ only by
    near-tie swaps, and the output is compared on the set the GPU used).
    Every row is compared; selections must list valid pages."""
    sel = np.ascontiguousarray(sel, np.int32)
    n_sel = np.ascontiguousarray(n_sel, np.int32)
    ps = sc.w.page_size
    for b, n in enumerate(sc.lengths):
        npg = -(-int(n) // ps)
        for h in range(sc.w.units):
            k = int(n_sel[b, h])
            assert 0 <= k <= sc.w.top_k and all(0 <= j < npg for j in sel[b, h, :k])
    z_ref, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    rtol, atol = (2e-2, 2e-3) if sc.w.dtype == BF16 else (1e-4, 1e-4)
    np.testing.assert_allclose(np.asarray(out, np.float64), out_ref, rtol=rtol, atol=atol)
    np.testing.assert_allclose(np.asarray(z, np.float64), z_ref, rtol=rtol, atol=atol)


U32 = 2.0 ** -24  # fp32 unit roundoff


def ulp(x: np.ndarray, dtype: int) -> np.ndarray:
    """Spacing of the storage dtype at |x| (bf16: 8 significant bits, fp32: 24)."""
    bits = 8 if dtype == BF16 else 24
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - bits + 1)


def bf16_midpoint_distance(x: np.ndarray) -> np.ndarray:
    """Distance of each real x to the nearest point where round-to-nearest
    into bf16 (8 significant bits) changes its result: the midpoints between
    neighbouring bf16 values (spacing halves below a power of two)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    lo = 2.0 ** e
    u = 2.0 ** (e - 7)                       # bf16 spacing in [2^e, 2^(e+1))
    frac = (a - lo) / u                      # position within the binade, in spacings
    d_in = np.abs(frac - np.floor(frac) - 0.5) * u
    d_below = (a - lo) + u / 4               # the midpoint just under 2^e (spacing u/2 there)
    return np.minimum(d_in, d_below)


def check_rounded_dot(got, ref, n_terms, mag, dtype, extra=0.0, exact=None):
    """A stored result of an n-term fp32 dot product against the oracle's
    correctly rounded one.

    Always: |got - ref| <= n*u*sum|terms| + extra + one storage ulp (both
    sides round once; the fp32 accumulation error bound).
    bf16 with ``exact`` (the real value the oracle rounded; NaN where it is
    not known): the GPU's fp32 value lies within n*u*sum|terms| of the exact
    one, so its bf16 rounding can differ from the correctly rounded value
    only where the exact value lies within that bound of a rounding
    midpoint; every mismatch elsewhere fails.  (Returns the mismatch count.)"""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    acc_bound = n_terms * U32 * mag + extra
    bound = acc_bound + ulp(np.maximum(np.abs(got), np.abs(ref)), dtype)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], ref[bad][:5], bound[bad][:5])
    mism = got != ref
    if exact is not None and mism.any():
        ex = np.broadcast_to(np.asarray(exact, np.float64), got.shape)[mism]
        ab = np.broadcast_to(np.asarray(acc_bound, np.float64), got.shape)[mism]
        known = np.isfinite(ex)
        dist = bf16_midpoint_distance(ex[known])
        # (1e-12 relative: the fp64 rounding of the exact value itself)
        far = dist > ab[known] + 1e-12 * np.abs(ex[known])
        assert not far.any(), ("mismatch away from a rounding midpoint", ex[known][far][:5],
                               got[mism][known][far][:5], ref[mism][known][far][:5], dist[far][:5])
    return int(mism.sum())


def _valid_slots(sc, page_table):
    """(page, slot) of every written token, and the tokens' Keys/Values in that order."""
    P, T, K, V = [], [], [], []
    ps = sc.w.page_size
    for b, n in enumerate(sc.lengths):
        for t in range(int(n)):
            P.append(page_table[b, t // ps])
            T.append(t % ps)
        K.append(sc.K[b][:int(n)])
        V.append(sc.V[b][:int(n)])
    return np.array(P), np.array(T), np.concatenate(K), np.concatenate(V)


def compare_written(sc, got, ora, got_page_table=None):
    """A GPU-written cache (host arrays K, Z, S, summ) against the oracle-written
    one: Keys bit for bit; latents and residuals within the fp32 accumulation
    bound plus one storage ulp of the oracle's correctly rounded values, and
    in bf16 different from them only where the exact value lies within that
    bound of a rounding midpoint; page sums equal to the fp32 slot-order
    sum of the GPU's own stored values.  got_page_table: the GPU's placement
    of the scenario's rows (default: the scenario's own)."""
    w = sc.w
    dt = w.dtype
    D, R, RK = w.head_dim, w.rank_v, w.rank_k
    gpt = sc.page_table if got_page_table is None else got_page_table
    P, T, Kt, Vt = _valid_slots(sc, sc.page_table)
    Pg, _, _, _ = _valid_slots(sc, gpt)
    # exact Keys, bit for bit
    assert np.array_equal(got["K"][Pg, :, T], ora.K[P, :, T])
    zg = synth.storage_to_f64(got["Z"][Pg, :, :, T], dt)   # [tokens][H][R]
    zo = synth.storage_to_f64(ora.Z[P, :, :, T], dt)
    sg = synth.storage_to_f64(got["S"][Pg, :, T], dt)      # [tokens][H][RK]
    so = synth.storage_to_f64(ora.S[P, :, T], dt)
    K = synth.storage_to_f64(Kt, dt)
    V = synth.storage_to_f64(Vt, dt)
    bf = dt == BF16
    mism = [0, 0]
    for g in range(w.n_kv_heads):
        B64 = sc.fac.B[g].astype(np.float64)
        P64 = sc.fac.P[g].astype(np.float64)
        Re64 = sc.fac.R_enc[g].astype(np.float64)
        B, Pm, Re = np.abs(B64), np.abs(P64), np.abs(Re64)
        # latent z = v.B: D terms; exact value v.B in fp64
        mism[0] += check_rounded_dot(zg[:, g], zo[:, g], D, np.abs(V[:, g]) @ B, dt,
                                     exact=V[:, g] @ B64 if bf else None)
        # residual s = (k - z~.P).R_enc: the latent's own difference propagates,
        # then R + D accumulated terms.  The exact residual is known where the
        # GPU stored the oracle's latent row (everywhere else: NaN, bound only).
        prop = (np.abs(zg[:, g] - zo[:, g]) @ Pm) @ Re
        mag = (np.abs(K[:, g]) + np.abs(zo[:, g]) @ Pm) @ Re
        ex = None
        if bf:
            ex = (K[:, g] - zo[:, g] @ P64) @ Re64
            ex[~np.all(zg[:, g] == zo[:, g], axis=1)] = np.nan
        mism[1] += check_rounded_dot(sg[:, g], so[:, g], D + R, mag, dt, extra=prop, exact=ex)
    if bf:
        n = zg.shape[0] * w.n_kv_heads
        print(f"[writer] bf16 values differing from the correctly rounded ones: latents {mism[0]} of {n * R}, "
              f"residuals {mism[1]} of {n * RK}", flush=True)
    # page sums: the fp32 sum of the GPU's own stored values, in slot order
    ps = w.page_size
    vz = synth.storage_to_f64(got["Z"], dt)
    vs = synth.storage_to_f64(got["S"], dt)
    for b, n in enumerate(sc.lengths):
        for j in range(-(-int(n) // ps)):
            p = gpt[b, j]
            cnt = min(ps, int(n) - j * ps)
            for g in range(w.n_kv_heads):
                x = np.concatenate([vz[p, g, :, :cnt].T, vs[p, g, :cnt, :]], axis=1)  # [cnt][R+RK]
                ref = x.sum(axis=0)
                bound = cnt * U32 * np.abs(x).sum(axis=0) + 1e-30
                assert np.all(np.abs(got["summ"][p, g] - ref) <= bound), (b, j, g)
