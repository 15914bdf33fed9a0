"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one part of the oracle to a closed form, a textbook routine, a
brute-force enumeration or an invariant the method must satisfy, chosen so
that a plausible slip (a dropped term, a transposed factor, a wrong index or
sign) fails at least one of them.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import cases
from tests.cases import small, make_scenario, to_f64
from workloads import synth
from workloads.configs import BF16, F32

oracle.build(force=False)


# ---- storage rounding ---------------------------------------------------------

def test_round_bf16_matches_torch_rne():
    """The oracle's bf16 rounding equals torch's fp32->bf16 round-to-nearest-even."""
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),     # subnormal range
        (rng.standard_normal(2000) * 3e38).astype(np.float32),      # near overflow
        np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -133, 2 ** -134,
                    3 * 2 ** -134, 0.0, -0.0, np.inf, -np.inf, 3.3895314e38]),
    ])
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_bf16(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, want)


def test_round_bf16_ties_to_even_on_exact_reals():
    # 1 + 2^-8 lies exactly between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert oracle.round_bf16(1 + 2 ** -8) == 0x3F80
    # 1 + 3*2^-8 lies between 1+2^-7 (odd) and 1+2^-6 (even)
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 0x3F82
    # just above the midpoint rounds up
    assert oracle.round_bf16(1 + 2 ** -8 + 2 ** -40) == 0x3F81


# ---- hand-derived worked example ------------------------------------------------

def test_hand_worked_example():
    """tests/golden/hand_two_pages.json: every value derived by hand."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_two_pages.json")))
    dm = g["dims"]
    for top_k, exp in (("1", g["expected_top1"]), ("2", g["expected_top2"])):
        d = oracle.Dims(batch=1, n_q_heads=1, n_kv_heads=1, head_dim=dm["head_dim"],
                        rank_v=dm["rank_v"], rank_k=dm["rank_k"], page_size=dm["page_size"],
                        d_model=dm["d_model"], top_k=int(top_k), max_pages=2, num_pages=2,
                        dtype=F32, scale=dm["scale"])
        fac = synth.Factors(mix=None, B=np.array([g["B"]], np.float32),
                            P=np.array([g["P"]], np.float32),
                            R_enc=np.array([g["R_enc"]], np.float32),
                            R_dec=np.array([g["R_dec"]], np.float32),
                            W_O=np.array(g["W_O"], np.float32))
        cache = oracle.Cache(d, np.array([[0, 1]], np.int32))
        k = np.array(g["k"], np.float32)[:, None, :]
        v = np.array(g["v"], np.float32)[:, None, :]
        oracle.write(d, fac, cache, 0, 0, k, v)
        np.testing.assert_array_equal(cache.summ[:, 0, :], np.array(g["expected_summ"], np.float32))
        W = oracle.fold(d, fac.B, fac.W_O)
        q = np.array([[g["q"]]], np.float32)
        sel, n_sel, scores = oracle.route(d, fac, cache, np.array([3], np.int32), q)
        np.testing.assert_allclose(scores[0, 0], g["expected_scores"], rtol=0, atol=1e-6)
        assert sel[0, 0].tolist() == exp["sel"]
        z, out = oracle.decode(d, W, cache, np.array([3], np.int32), q, sel, n_sel)
        e = math.e
        zexp = [eval(s, {"e": e}) for s in exp["zhat"]]
        oexp = [eval(s, {"e": e}) for s in exp["out"]]
        np.testing.assert_allclose(z[0, 0], zexp, rtol=1e-7)
        np.testing.assert_allclose(out[0], oexp, rtol=1e-7)


# ---- P-1: reduces to textbook dense attention ----------------------------------

@pytest.mark.parametrize("dtype", [F32])
def test_full_rank_all_pages_is_dense_attention(dtype):
    """r = d_h, orthonormal B, every page selected: out = softmax(qK^T/sqrt(d)) V W_O."""
    w = small("p1", 101, rank_v=16, rank_k=4, top_k=16, dtype=dtype)
    sc = make_scenario(w, lengths=[37, 22])
    sel, n_sel, _ = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    assert n_sel.tolist() == [[10, 10], [6, 6]]
    z, out = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    G = w.group
    WO = to_f64(sc.fac.W_O, dtype)
    for b, n in enumerate(sc.lengths):
        ref = np.zeros(w.d_model)
        for h in range(w.n_q_heads):
            g = h // G
            K = to_f64(sc.K[b][:, g], dtype)
            V = to_f64(sc.V[b][:, g], dtype)
            qh = to_f64(sc.q[b, h], dtype)
            p = cases.softmax(K @ qh / math.sqrt(w.head_dim))
            ref += (p @ V) @ WO[h * w.head_dim:(h + 1) * w.head_dim]
        np.testing.assert_allclose(out[b], ref, rtol=1e-5, atol=1e-6)


# ---- P-12: writer against numpy ---------------------------------------------------

def _page_tokens(sc, b, g):
    """Stored (z~, s~, k) of sequence b, head g in token order, from the oracle cache."""
    ps, n = sc.w.page_size, int(sc.lengths[b])
    zs, ss, ks = [], [], []
    for t in range(n):
        p = sc.page_table[b, t // ps]
        zs.append(sc.cache.Z[p, g, :, t % ps])
        ss.append(sc.cache.S[p, g, t % ps, :])
        ks.append(sc.cache.K[p, g, t % ps, :])
    return np.array(zs), np.array(ss), np.array(ks)


def test_writer_fp32_matches_numpy():
    w = small("p12", 112, dtype=F32)
    sc = make_scenario(w, lengths=[37, 22])
    for b in range(2):
        for g in range(w.n_kv_heads):
            z, s, k = _page_tokens(sc, b, g)
            V = sc.V[b][:, g].astype(np.float64)
            K = sc.K[b][:, g].astype(np.float64)
            zref = (V @ sc.fac.B[g].astype(np.float64)).astype(np.float32)
            assert np.array_equal(z, zref)
            e = K - z.astype(np.float64) @ sc.fac.P[g].astype(np.float64)
            sref = (e @ sc.fac.R_enc[g].astype(np.float64)).astype(np.float32)
            assert np.array_equal(s, sref)
            assert np.array_equal(k, sc.K[b][:, g])


def test_writer_bf16_within_one_ulp_of_numpy():
    w = small("p12b", 113, dtype=BF16, head_dim=64, rank_v=16, rank_k=8, page_size=16, ctx=200)
    sc = make_scenario(w, lengths=[200, 77])
    tot = mism = 0
    for b in range(2):
        for g in range(w.n_kv_heads):
            z, s, k = _page_tokens(sc, b, g)
            V = to_f64(sc.V[b][:, g], BF16)
            zref = synth.to_storage(V @ sc.fac.B[g].astype(np.float64), BF16)
            diff = np.abs(z.astype(np.int32) - zref.astype(np.int32))
            assert diff.max() <= 1
            tot += diff.size
            mism += int((diff > 0).sum())
            # residual from the stored latent
            e = to_f64(sc.K[b][:, g], BF16) - to_f64(z, BF16) @ sc.fac.P[g].astype(np.float64)
            sref = synth.to_storage(e @ sc.fac.R_enc[g].astype(np.float64), BF16)
            assert np.abs(s.astype(np.int32) - sref.astype(np.int32)).max() <= 1
    assert mism <= 1e-3 * tot


# ---- P-2 / P-3: router scores ------------------------------------------------------

def _numpy_page_scores(sc, b, g, ktilde):
    """scale * max_h q_h . mean_t ktilde_t per logical page (numpy fp64)."""
    w, ps, n = sc.w, sc.w.page_size, int(sc.lengths[b])
    G = w.group
    qs = to_f64(sc.q[b, g * G:(g + 1) * G], w.dtype)
    out = []
    for j in range(-(-n // ps)):
        kt = ktilde[j * ps:min(n, (j + 1) * ps)].mean(axis=0)
        out.append(max(float(qh @ kt) for qh in qs) * w.softmax_scale)
    return np.array(out)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_route_scores_are_mean_predicted_key(dtype):
    """Page score from the page sums == mean over its tokens of z~P + s~R_dec."""
    w = small("p2", 102, dtype=dtype, top_k=4)
    sc = make_scenario(w, lengths=[37, 22])
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    for b in range(2):
        for g in range(w.n_kv_heads):
            z, s, _ = _page_tokens(sc, b, g)
            kt = to_f64(z, dtype) @ sc.fac.P[g].astype(np.float64) + \
                to_f64(s, dtype) @ sc.fac.R_dec[g].astype(np.float64)
            ref = _numpy_page_scores(sc, b, g, kt)
            npg = len(ref)
            np.testing.assert_allclose(scores[b, g, :npg], ref, rtol=1e-5, atol=1e-6)
            assert np.all(np.isneginf(scores[b, g, npg:]))
            assert n_sel[b, g] == min(w.top_k, npg)
            cases.check_selection_valid(ref, sel[b, g, :n_sel[b, g]], n_sel[b, g], 1e-5)


def test_route_with_exact_key_residual_scores_raw_keys():
    """r_k = d_h and R_enc = R_dec = I: the predicted Key is the Key itself."""
    w = small("p3", 103, rank_k=16, top_k=3)
    fac = synth.make_factors(w)
    eye = np.broadcast_to(np.eye(16, dtype=np.float32), (w.n_kv_heads, 16, 16)).copy()
    fac.R_enc, fac.R_dec = eye, eye.copy()
    sc = make_scenario(w, lengths=[37, 22], write=False)
    sc.fac = fac
    cache = oracle.Cache(sc.d, sc.page_table)
    for b in range(2):
        oracle.write(sc.d, fac, cache, b, 0, sc.K[b], sc.V[b])
    sel, n_sel, scores = oracle.route(sc.d, fac, cache, sc.lengths, sc.q)
    for b in range(2):
        for g in range(w.n_kv_heads):
            ref = _numpy_page_scores(sc, b, g, sc.K[b][:, g].astype(np.float64))
            np.testing.assert_allclose(scores[b, g, :len(ref)], ref, rtol=1e-5, atol=1e-6)
            cases.check_selection_valid(ref, sel[b, g, :n_sel[b, g]], n_sel[b, g], 1e-5)


# ---- P-4: selection rule, brute force, exact ties ---------------------------------

def _hand_cache(n_pages, ps, G, values):
    """A cache whose page scores are exactly `values[h][j]` for query head h.

    d_h = 4, r = r_k = 2, scale 1; query head h is the unit vector e_h, P maps
    e_0 -> latent 0 and e_1 -> latent 1, R_dec maps e_2, e_3 -> residual 0, 1.
    The page sums are values * count, so score_h(j) = values[h][j] exactly.
    """
    d = oracle.Dims(batch=1, n_q_heads=G, n_kv_heads=1, head_dim=4, rank_v=2, rank_k=2,
                    page_size=ps, d_model=1, top_k=1, max_pages=n_pages, num_pages=n_pages,
                    dtype=F32, scale=1.0)
    P = np.zeros((1, 2, 4), np.float32); P[0, 0, 0] = P[0, 1, 1] = 1
    Rd = np.zeros((1, 2, 4), np.float32); Rd[0, 0, 2] = Rd[0, 1, 3] = 1
    fac = synth.Factors(mix=None, B=None, P=P, R_enc=None, R_dec=Rd, W_O=None)
    cache = oracle.Cache(d, np.arange(n_pages, dtype=np.int32)[None])
    q = np.zeros((1, G, 4), np.float32)
    for h in range(G):
        q[0, h, h] = 1
    return d, fac, cache, q


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    ps = 4
    G = 1 + seed % 4
    n = int(rng.integers(0, 60))
    npg = -(-n // ps)
    n_pages = max(npg, 1)
    vals = rng.integers(-3, 4, size=(G, n_pages)).astype(np.float64)
    d, fac, cache, q = _hand_cache(n_pages, ps, G, vals)
    for j in range(npg):
        cnt = min(ps, n - j * ps)
        for h in range(G):
            # head h's value sits in latent h (h<2) or residual h-2
            cache.summ[j, 0, h] = vals[h, j] * cnt
    for top_k in (1, 3, 5, 16):
        d.top_k = top_k
        sel, n_sel, scores = oracle.route(d, fac, cache, np.array([n], np.int32), q)
        agg = vals.max(axis=0)[:npg]
        keff = min(top_k, npg)
        assert n_sel[0, 0] == keff
        assert sel[0, 0, :keff].tolist() == cases.brute_topk(agg, keff)
        assert (sel[0, 0, keff:] == -1).all()
        np.testing.assert_array_equal(scores[0, 0, :npg], agg.astype(np.float32))


@pytest.mark.parametrize("seed", range(10))
def test_forced_pages_brute_force(seed):
    """Pages kept at either end of the sequence (sink_pages, local_pages)
    rank above every score, among themselves by page; the rest by score,
    ties to the smaller page."""
    rng = np.random.default_rng(100 + seed)
    ps, G = 4, 1 + seed % 3
    n = int(rng.integers(1, 60))
    npg = -(-n // ps)
    vals = rng.integers(-3, 4, size=(G, npg)).astype(np.float64)
    d, fac, cache, q = _hand_cache(npg, ps, G, vals)
    for j in range(npg):
        cnt = min(ps, n - j * ps)
        for h in range(G):
            cache.summ[j, 0, h] = vals[h, j] * cnt
    agg = vals.max(axis=0)
    for sink, local, top_k in ((1, 0, 3), (0, 2, 3), (2, 2, 5), (3, 3, 4), (1, 1, 16), (0, 0, 5)):
        d.top_k, d.sink_pages, d.local_pages = top_k, sink, local
        sel, n_sel, scores = oracle.route(d, fac, cache, np.array([n], np.int32), q)
        forced = [j for j in range(npg) if j < sink or j >= npg - local]
        rest = sorted((j for j in range(npg) if j not in forced), key=lambda j: (-agg[j], j))
        keff = min(top_k, npg)
        want = sorted((forced + rest)[:keff])
        assert n_sel[0, 0] == keff
        assert sel[0, 0, :keff].tolist() == want, (sink, local, top_k)
        np.testing.assert_array_equal(scores[0, 0, :npg], agg.astype(np.float32))  # scores unchanged


@pytest.mark.parametrize("seed", range(6))
def test_group_mean_brute_force(seed):
    """group_mean: a page's score is the mean of its query heads' scores."""
    rng = np.random.default_rng(200 + seed)
    ps, G = 4, 2 + seed % 3
    n = int(rng.integers(1, 60))
    npg = -(-n // ps)
    vals = rng.integers(-3, 4, size=(G, npg)).astype(np.float64)
    d, fac, cache, q = _hand_cache(npg, ps, G, vals)
    for j in range(npg):
        cnt = min(ps, n - j * ps)
        for h in range(G):
            cache.summ[j, 0, h] = vals[h, j] * cnt
    d.group_mean = 1
    for top_k in (1, 3, 16):
        d.top_k = top_k
        sel, n_sel, scores = oracle.route(d, fac, cache, np.array([n], np.int32), q)
        mean = vals.mean(axis=0)
        np.testing.assert_allclose(scores[0, 0, :npg], mean, rtol=1e-6, atol=1e-6)
        keff = min(top_k, npg)
        assert sel[0, 0, :keff].tolist() == cases.brute_topk(scores[0, 0, :npg].astype(np.float64), keff)


# ---- head_select: every query head selects its own pages (routing variant) -----

@pytest.mark.parametrize("seed", range(8))
def test_head_select_brute_force(seed):
    """Each query head's scores are its own page values and its selection the
    brute-force top-k of them (ties to the smaller page, forced pages first)."""
    rng = np.random.default_rng(300 + seed)
    ps, G = 4, 2 + seed % 3
    n = int(rng.integers(1, 60))
    npg = -(-n // ps)
    vals = rng.integers(-3, 4, size=(G, npg)).astype(np.float64)
    d, fac, cache, q = _hand_cache(npg, ps, G, vals)
    for j in range(npg):
        cnt = min(ps, n - j * ps)
        for h in range(G):
            cache.summ[j, 0, h] = vals[h, j] * cnt
    d.head_select = 1
    d.sink_pages, d.local_pages = seed % 2, (seed // 2) % 2
    for top_k in (1, 3, 16):
        d.top_k = top_k
        sel, n_sel, scores = oracle.route(d, fac, cache, np.array([n], np.int32), q)
        assert sel.shape == (1, G, top_k) and n_sel.shape == (1, G)
        keff = min(top_k, npg)
        for h in range(G):
            np.testing.assert_array_equal(scores[0, h, :npg], vals[h].astype(np.float32))
            forced = [j for j in range(npg) if j < d.sink_pages or j >= npg - d.local_pages]
            rest = [j for j in sorted(range(npg), key=lambda j: (-vals[h, j], j)) if j not in forced]
            assert n_sel[0, h] == keff
            assert sel[0, h, :keff].tolist() == sorted((forced + rest)[:keff])
            assert (sel[0, h, keff:] == -1).all()


def test_head_select_decode_brute_force():
    """Per-head selection, then each query head's latent from a numpy softmax
    over the tokens of its own pages and the projection of all heads."""
    w = small("hs", 131, dtype=F32, top_k=3, head_select=1)
    sc = make_scenario(w, lengths=[37, 22])
    sel, n_sel, _ = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    assert sel.shape == (2, w.n_q_heads, w.top_k)
    z, out = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    G, ps = w.group, w.page_size
    differs = False
    for b in range(2):
        n = int(sc.lengths[b])
        for h in range(w.n_q_heads):
            g = h // G
            pages = sel[b, h, :n_sel[b, h]].tolist()
            differs |= pages != sel[b, g * G, :n_sel[b, g * G]].tolist()
            toks = [t for j in pages for t in range(j * ps, min(n, (j + 1) * ps))]
            K = to_f64(sc.K[b][toks, g], w.dtype)
            zt = np.stack([to_f64(sc.cache.Z[sc.page_table[b, t // ps], g, :, t % ps], w.dtype) for t in toks])
            p = cases.softmax(K @ to_f64(sc.q[b, h], w.dtype) * w.softmax_scale)
            np.testing.assert_allclose(z[b, h], p @ zt, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out[b], z[b].reshape(-1) @ to_f64(sc.W_ofT, w.dtype).T, rtol=1e-12, atol=1e-12)
    assert differs, "the case should give some heads of a group different pages"


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_head_select_scores_max_to_the_group_score(dtype):
    """The per-head scores' max over a group is the group score, bit for bit
    (fp32 rounding is monotone); with one query head per KV head both
    routings select the same pages and decode the same output."""
    w = small("hm", 132, dtype=dtype, top_k=4)
    sc = make_scenario(w, lengths=[37, 22])
    _, _, grp = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    sc.d.head_select = 1
    _, _, per = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    G = w.group
    for g in range(w.n_kv_heads):
        assert np.array_equal(per[:, g * G:(g + 1) * G].max(axis=1), grp[:, g])
    w1 = small("h1", 133, dtype=dtype, n_q_heads=2, n_kv_heads=2, top_k=4)
    sc1 = make_scenario(w1, lengths=[37, 22])
    res = []
    for hs in (0, 1):
        sc1.d.head_select = hs
        sel, n_sel, scores = oracle.route(sc1.d, sc1.fac, sc1.cache, sc1.lengths, sc1.q)
        res.append((sel, n_sel, scores) + oracle.decode(sc1.d, sc1.W_ofT, sc1.cache, sc1.lengths, sc1.q, sel, n_sel))
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_topk_all_equal_takes_first_pages():
    d, fac, cache, q = _hand_cache(10, 4, 1, np.zeros((1, 10)))
    cache.summ[:, 0, 0] = 8.0      # every score 2.0
    d.top_k = 4
    sel, n_sel, _ = oracle.route(d, fac, cache, np.array([40], np.int32), q)
    assert sel[0, 0].tolist() == [0, 1, 2, 3]


def test_topk_negative_zero_ties_positive_zero():
    d, fac, cache, q = _hand_cache(3, 4, 1, np.zeros((1, 3)))
    cache.summ[0, 0, 0] = -0.0
    cache.summ[1, 0, 0] = 0.0
    cache.summ[2, 0, 0] = -1.0
    d.top_k = 1
    sel, _, _ = oracle.route(d, fac, cache, np.array([12], np.int32), q)
    assert sel[0, 0].tolist() == [0]


def test_empty_sequence():
    w = small("p19", 119, top_k=3)
    sc = make_scenario(w, lengths=[0, 9])
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    assert n_sel[0].tolist() == [0, 0] and (sel[0] == -1).all()
    z, out = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    assert (z[0] == 0).all() and (out[0] == 0).all()
    assert np.abs(out[1]).max() > 0


# ---- P-5: weights sum to one -------------------------------------------------------

@pytest.mark.parametrize("dtype", [F32, BF16])
def test_constant_latents_give_that_latent(dtype):
    """If every stored latent is the same vector c, the weighted sum is c."""
    w = small("p5", 105, dtype=dtype, top_k=5)
    sc = make_scenario(w, lengths=[37, 22])
    c = synth.to_storage(np.array([0.5, -1.25, 2.0, 3.0]), dtype)
    sc.cache.Z[...] = c[None, None, :, None]
    sel, n_sel, _ = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    z, out = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    cf = to_f64(c, dtype)
    np.testing.assert_allclose(z, np.broadcast_to(cf, z.shape), rtol=0, atol=1e-14)
    W = to_f64(sc.W_ofT, dtype)
    ref = np.tile(cf, w.n_q_heads) @ W.T
    np.testing.assert_allclose(out, np.broadcast_to(ref, out.shape), rtol=1e-12, atol=1e-14)


# ---- P-6: physical placement does not matter ---------------------------------------

def _permuted_copy(sc, seed):
    pt2 = synth.permute_pool(sc.page_table, sc.num_pages, seed)
    c2 = oracle.Cache(sc.d, pt2)
    for b in range(sc.page_table.shape[0]):
        for j in range(sc.page_table.shape[1]):
            p, p2 = sc.page_table[b, j], pt2[b, j]
            if p < 0:
                continue
            c2.K[p2], c2.Z[p2], c2.S[p2], c2.summ[p2] = sc.cache.K[p], sc.cache.Z[p], \
                sc.cache.S[p], sc.cache.summ[p]
    return c2


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_page_permutation_bit_identical(dtype):
    w = small("p6", 106, dtype=dtype, top_k=3)
    sc = make_scenario(w, lengths=[37, 22])
    c2 = _permuted_copy(sc, 5)
    r1 = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    r2 = oracle.route(sc.d, sc.fac, c2, sc.lengths, sc.q)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)
    o1 = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, r1[0], r1[1])
    o2 = oracle.decode(sc.d, sc.W_ofT, c2, sc.lengths, sc.q, r1[0], r1[1])
    for a, b in zip(o1, o2):
        assert np.array_equal(a, b)


# ---- P-7: unused slots are never read --------------------------------------------

@pytest.mark.parametrize("dtype", [F32, BF16])
def test_poisoned_unused_slots_do_not_change_results(dtype):
    w = small("p7", 107, dtype=dtype, top_k=3)
    poison = np.float32(np.nan) if dtype == F32 else np.uint16(0x7FC0)
    clean = make_scenario(w, lengths=[37, 22], fill=0)
    dirty = make_scenario(w, lengths=[37, 22], fill=poison)
    # pool pages nobody maps and page sums nobody wrote
    dirty.cache.summ[...] = np.where(clean.cache.summ == 0, np.nan, dirty.cache.summ)
    r1 = oracle.route(clean.d, clean.fac, clean.cache, clean.lengths, clean.q)
    r2 = oracle.route(dirty.d, dirty.fac, dirty.cache, dirty.lengths, dirty.q)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])
    o1 = oracle.decode(clean.d, clean.W_ofT, clean.cache, clean.lengths, clean.q, r1[0], r1[1])
    o2 = oracle.decode(dirty.d, dirty.W_ofT, dirty.cache, dirty.lengths, dirty.q, r1[0], r1[1])
    assert np.all(np.isfinite(o2[1]))
    assert np.array_equal(o1[1], o2[1]) and np.array_equal(o1[0], o2[0])


# ---- P-8: every page selected == dense attention over the stored cache --------------

@pytest.mark.parametrize("dtype", [F32, BF16])
def test_all_pages_is_dense_attention_over_latents(dtype):
    w = small("p8", 108, dtype=dtype, top_k=10)
    sc = make_scenario(w, lengths=[37, 22])
    sel, n_sel = cases.all_pages_selection(sc.lengths, w.n_kv_heads, w.top_k, w.page_size)
    z, out = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    W = to_f64(sc.W_ofT, dtype)
    for b in range(2):
        zrow = []
        for h in range(w.n_q_heads):
            g = h // w.group
            zt, _, k = _page_tokens(sc, b, g)
            p = cases.softmax(to_f64(k, dtype) @ to_f64(sc.q[b, h], dtype) * w.softmax_scale)
            zrow.append(p @ to_f64(zt, dtype))
        zrow = np.concatenate(zrow)
        np.testing.assert_allclose(z[b].ravel(), zrow, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(out[b], W @ zrow, rtol=1e-12, atol=1e-13)


# ---- P-9 / P-10 / P-11: prefill, chunking, append ----------------------------------

def _prefill_case(dtype):
    w = small("p9", 109, dtype=dtype, batch=1, top_k=8, ctx=23)
    sc = make_scenario(w, lengths=[23], write=False)
    qp = synth.to_storage(np.random.default_rng(3).standard_normal((23, w.n_q_heads, w.head_dim)), dtype)
    return w, sc, qp


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_prefill_row_equals_decode_at_that_length(dtype):
    w, sc, qp = _prefill_case(dtype)
    cache = oracle.Cache(sc.d, sc.page_table)
    W = oracle.fold(sc.d, sc.fac.B, sc.fac.W_O)
    zp, op = oracle.prefill(sc.d, sc.fac, W, cache, 0, 0, qp, sc.K[0], sc.V[0])
    for p in range(23):
        L = np.array([p + 1], np.int32)
        sel, n_sel = cases.all_pages_selection(L, w.n_kv_heads, w.top_k, w.page_size)
        zd, od = oracle.decode(sc.d, W, cache, L, qp[p:p + 1], sel, n_sel)
        np.testing.assert_allclose(zp[p], zd[0], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(op[p], od[0], rtol=1e-12, atol=1e-15)
    # the first query sees only itself: its latent is exactly the stored one
    ps = w.page_size
    for h in range(w.n_q_heads):
        g = h // w.group
        np.testing.assert_array_equal(zp[0, h], to_f64(cache.Z[sc.page_table[0, 0], g, :, 0], dtype))


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_chunked_prefill_and_appends_equal_one_shot(dtype):
    w, sc, qp = _prefill_case(dtype)
    W = oracle.fold(sc.d, sc.fac.B, sc.fac.W_O)
    one = oracle.Cache(sc.d, sc.page_table)
    z1, o1 = oracle.prefill(sc.d, sc.fac, W, one, 0, 0, qp, sc.K[0], sc.V[0])
    chunked = oracle.Cache(sc.d, sc.page_table)
    zs, os_ = [], []
    for a, b in ((0, 7), (7, 16), (16, 23)):
        z, o = oracle.prefill(sc.d, sc.fac, W, chunked, 0, a, qp[a:b], sc.K[0][a:b], sc.V[0][a:b])
        zs.append(z); os_.append(o)
    appended = oracle.Cache(sc.d, sc.page_table)
    for t in range(23):
        oracle.write(sc.d, sc.fac, appended, 0, t, sc.K[0][t:t + 1], sc.V[0][t:t + 1])
    for c in (chunked, appended):
        for n in ("K", "Z", "S", "summ"):
            assert np.array_equal(getattr(c, n), getattr(one, n)), n
    np.testing.assert_array_equal(np.concatenate(zs), z1)
    np.testing.assert_array_equal(np.concatenate(os_), o1)


# ---- P-13: grouped-query routing ---------------------------------------------------

def test_gqa_identical_heads_route_like_one_head():
    w = small("p13", 113, n_q_heads=4, n_kv_heads=1, top_k=3)
    sc = make_scenario(w, lengths=[37, 22])
    q4 = np.repeat(sc.q[:, :1], 4, axis=1)
    s4 = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, q4)
    w1 = w.with_(n_q_heads=1)
    d1 = oracle.Dims.of(w1, batch=2, num_pages=sc.num_pages)
    s1 = oracle.route(d1, sc.fac, sc.cache, sc.lengths, np.ascontiguousarray(sc.q[:, :1]))
    for a, b in zip(s4, s1):
        assert np.array_equal(a, b)


# ---- fold ------------------------------------------------------------------------

def test_fold_is_basis_transpose_times_output_slice():
    w = small("fold", 114, dtype=F32)
    fac = synth.make_factors(w)
    d = oracle.Dims.of(w, batch=1, num_pages=1)
    W = oracle.fold(d, fac.B, fac.W_O)
    G, D, R = w.group, w.head_dim, w.rank_v
    for h in range(w.n_q_heads):
        ref = fac.B[h // G].astype(np.float64).T @ fac.W_O[h * D:(h + 1) * D].astype(np.float64)
        np.testing.assert_array_equal(W[:, h * R:(h + 1) * R], ref.T.astype(np.float32))


# ---- P-14: byte accounting ------------------------------------------------------

def test_kv_size_formula_reproduces_70b_128k_figure():
    """A 70B model (80 layers, 8 KV heads of 128) at 128K tokens needs > 40 GB of fp16 KV."""
    from workloads.accounting import dense_kv_bytes
    b = dense_kv_bytes(80, 8, 128, 131072, 2)
    assert b == 42_949_672_960 and b > 40e9


def test_step_bytes_of_the_32k_share():
    from workloads import accounting, configs
    w = configs.get("llama8b_32k")
    sb = accounting.decode_step_bytes(w, [w.ctx] * w.batch)
    assert sb.keys == 16 * 64 * 64 * 128 * 2
    assert sb.latents == 16 * 64 * 64 * 32 * 2
    assert sb.summaries == 16 * 512 * 48 * 4
    assert sb.total == 23_973_376
