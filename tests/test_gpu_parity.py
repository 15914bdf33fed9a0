"""GPU parity: every entry point of the C-ABI library against the CPU oracle.

Inputs are the seeded synthetic workloads (tests/cases.py); the oracle never
receives anything the GPU produced.  Where a test wants identical cache
contents, the oracle's cache is uploaded to the GPU.  Tolerances: selected
page sets identical up to swaps of pages whose oracle fp32 scores differ by
less than 1e-5 relative; outputs within rtol 2e-2 / atol 2e-3 for bf16
storage (fp32 accumulation) and 1e-4 for fp32 storage.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import cases
from tests.cases import small
from workloads import configs, synth
from workloads.configs import BF16, F32

pytestmark = pytest.mark.gpu

gc = None


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    global gc
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    from tests import gpu_cases
    gc = gpu_cases
    oracle.build(force=False)


# Shapes: the headline geometry (d_h 128, pages of 64, r 32, GQA 4:1) at short
# contexts, wider groups with two KV heads and r 48 (pages of 32), head_dim
# 64, fp32 storage, and bf16 pages of 16 (plain kernels).  Lengths mix
# ragged tails, an exactly full page and a single token.
CASES = {
    "g4_d128_p64": (configs.get("llama8b_32k").with_(name="g4", cfg_id=201, batch=3, top_k=5,
                                                     d_model=256), [700, 64, 130]),
    "g8_2kv_r48_p32": (small("g8", 202, batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128,
                             page_size=32, rank_v=48, rank_k=16, top_k=7, d_model=192,
                             dtype=BF16, ctx=513), [513, 200]),
    "g1_d64": (small("g1", 203, batch=2, n_q_heads=2, n_kv_heads=2, head_dim=64, page_size=64,
                     rank_v=16, rank_k=8, top_k=3, d_model=128, dtype=BF16, ctx=300), [300, 1]),
    "tiny_f32": (configs.get("tiny_f32"), [1024]),
    "f32_p16_g2": (small("f32g2", 204, batch=2, n_q_heads=2, n_kv_heads=1, head_dim=64,
                         page_size=16, rank_v=16, rank_k=8, top_k=4, d_model=96, dtype=F32, ctx=100),
                   [100, 33]),
    "bf16_p16": (small("p16", 205, batch=2, n_q_heads=2, n_kv_heads=1, head_dim=64,
                       page_size=16, rank_v=16, rank_k=8, top_k=4, d_model=64, dtype=BF16, ctx=100),
                 [100, 33]),
    # forced pages: the first and the last two of every sequence are always kept
    "g4_forced": (configs.get("llama8b_32k").with_(name="g4f", cfg_id=207, batch=3, top_k=6, d_model=256,
                                                   sink_pages=1, local_pages=2), [700, 64, 130]),
    # the group's mean score instead of its max, alone and with forced pages
    "g4_mean": (configs.get("llama8b_32k").with_(name="g4m", cfg_id=208, batch=3, top_k=5, d_model=256,
                                                 group_mean=1), [700, 64, 130]),
    "g8_mean_forced": (small("g8mf", 209, batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128, page_size=32,
                             rank_v=48, rank_k=16, top_k=7, d_model=192, dtype=BF16, ctx=513, group_mean=1,
                             sink_pages=1, local_pages=1), [513, 200]),
    # one page per pair (below the sorting network's range), and more pages
    # than one wave's network keeps (the router's radix selection) at <= 512 pages
    "g4_k1": (configs.get("llama8b_32k").with_(name="g4k1", cfg_id=210, batch=3, top_k=1, d_model=256),
              [700, 64, 130]),
    "g4_k100": (configs.get("llama8b_32k").with_(name="g4k100", cfg_id=211, batch=3, top_k=100, d_model=256),
                [8000, 64, 6500]),
    # many pairs: 96 rows x 2 KV heads, lengths from the generator up to 600
    "wide_b96": (small("wb96", 212, batch=96, n_q_heads=8, n_kv_heads=2, head_dim=128, page_size=64,
                       rank_v=32, rank_k=16, top_k=4, d_model=256, dtype=BF16, ctx=600),
                 [(37 * i * i + 11 * i) % 600 + 1 for i in range(96)]),
    # contraction of 8 query heads x r 48 = 384 in the fused merge-projection
    # (above 256, within its 512 limit), three attention splits per pair
    "g4_2kv_r48_k384": (small("k384", 213, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, page_size=64,
                              rank_v=48, rank_k=16, top_k=12, d_model=256, dtype=BF16, ctx=1500),
                        [1500, 700]),
    # batches past one MFMA row tile: the merge-projection in 16-row tiles,
    # the last tile partly filled (24 and 40 rows)
    "b24_rows": (small("b24", 214, batch=24, n_q_heads=8, n_kv_heads=2, head_dim=128, page_size=64, rank_v=32,
                       rank_k=16, top_k=6, d_model=256, dtype=BF16, ctx=700),
                 [(53 * i + 17) % 700 + 1 for i in range(24)]),
    "b40_rows": (small("b40", 215, batch=40, n_q_heads=4, n_kv_heads=1, head_dim=128, page_size=32, rank_v=32,
                       rank_k=16, top_k=9, d_model=128, dtype=BF16, ctx=900),
                 [(71 * i + 5) % 900 + 1 for i in range(40)]),
    # 16-row tiles with more attention splits (10) than the row-tile merge
    # requests together (8), and ragged lengths below top_k pages
    "b20_k40": (small("b20", 216, batch=20, n_q_heads=4, n_kv_heads=1, head_dim=128, page_size=64, rank_v=32,
                      rank_k=16, top_k=40, d_model=128, dtype=BF16, ctx=3000),
                [(97 * i + 13) % 3000 + 1 for i in range(20)]),
    "ragged_permuted": (configs.get("ragged_mix").with_(name="rg", cfg_id=206, batch=5,
                                                        length_range=(1, 3000), top_k=16,
                                                        d_model=256),
                        None),
}


def scenario(name, **kw):
    w, lengths = CASES[name]
    return cases.make_scenario(w, lengths=lengths, **kw)


from tests.cases import U32, check_rounded_dot, compare_written  # noqa: E402


@pytest.mark.parametrize("name", sorted(CASES))
def test_fold_matches_oracle(name):
    sc = scenario(name)
    g = gc.upload(sc, cache=True)
    got = gc.host(g.f.W_ofT)
    w = sc.w
    WO64 = synth.storage_to_f64(sc.fac.W_O, w.dtype)
    WO = np.abs(WO64)
    mag = np.zeros((w.d_model, w.n_q_heads * w.rank_v))
    exact = np.zeros_like(mag)
    for h in range(w.n_q_heads):
        B64 = sc.fac.B[h // w.group].astype(np.float64)                   # [D][R]
        rows = slice(h * w.head_dim, (h + 1) * w.head_dim)
        mag[:, h * w.rank_v:(h + 1) * w.rank_v] = (np.abs(B64).T @ WO[rows]).T
        exact[:, h * w.rank_v:(h + 1) * w.rank_v] = (B64.T @ WO64[rows]).T
    check_rounded_dot(synth.storage_to_f64(got, w.dtype), synth.storage_to_f64(sc.W_ofT, w.dtype),
                      w.head_dim, mag, w.dtype, exact=exact if w.dtype == BF16 else None)


@pytest.mark.parametrize("name", sorted(CASES))
def test_writer_matches_oracle(name):
    sc = scenario(name)
    g = gc.upload(sc)
    gc.write_all(g, sc, chunk=97)  # chunks straddle page boundaries
    torch.cuda.synchronize()
    compare_written(sc, gc.cache_host(g), sc.cache)


@pytest.mark.parametrize("name", ["g4_d128_p64", "tiny_f32", "ragged_permuted"])
def test_appends_equal_one_chunk_write(name):
    sc = scenario(name)
    a = gc.upload(sc)
    gc.write_all(a, sc)
    b = gc.upload(sc)
    gc.write_all(b, sc, upto_last=True, chunk=50)
    gc.append_last(b, sc)
    gc.append_last(b, sc)  # rewriting the same position is idempotent
    torch.cuda.synchronize()
    ca, cb = gc.cache_host(a), gc.cache_host(b)
    for k in ca:
        assert np.array_equal(ca[k], cb[k]), k


@pytest.mark.parametrize("pages_per_wg", [None, 3])
@pytest.mark.parametrize("name", sorted(CASES))
def test_route_matches_oracle(name, pages_per_wg, monkeypatch):
    """The default scoring plan, and one of a few pages per scoring
    workgroup (ragged last range): same bits either way."""
    sc = scenario(name)
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    g = gc.upload(sc, cache=True)
    single = gc.route(g)
    if pages_per_wg is None:
        gs, gn, gscores = single
    else:
        monkeypatch.setenv("BASISKV_SCORE_PAGES_PER_WG", str(pages_per_wg))
        gs, gn, gscores = gc.route(g)
        gs2, gn2, gscores2 = gc.route(g)
        assert np.array_equal(gs, gs2) and np.array_equal(gn, gn2)
        assert np.array_equal(gs, single[0]) and np.array_equal(gn, single[1])
        for b, n in enumerate(sc.lengths):
            npg = -(-int(n) // sc.w.page_size)
            assert np.array_equal(gscores[b, :, :npg], single[2][b, :, :npg])
    assert np.array_equal(gn, n_sel)
    for b, n in enumerate(sc.lengths):
        npg = -(-int(n) // sc.w.page_size)
        for h in range(sc.w.n_kv_heads):
            k = int(n_sel[b, h])
            np.testing.assert_allclose(gscores[b, h, :npg], scores[b, h, :npg], rtol=1e-5,
                                       atol=1e-5 * max(1.0, float(np.abs(scores[b, h, :npg]).max(initial=0))))
            forced = [j for j in range(npg) if j < sc.w.sink_pages or j >= npg - sc.w.local_pages]
            ranked = scores[b, h, :npg].astype(np.float64).copy()
            ranked[forced] = np.inf  # forced pages rank above every score
            cases.check_selection_valid(ranked, gs[b, h, :k], k, 1e-5)
            assert set(forced[:k]) <= set(gs[b, h, :k].tolist())
            assert (gs[b, h, k:] == -1).all()


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_matches_oracle(name):
    sc = scenario(name)
    sel, n_sel, _ = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    z_ref, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    g = gc.upload(sc, cache=True, W_ofT=sc.W_ofT)
    z, out = gc.decode(g, sel, n_sel)
    rtol, atol = gc.tol(sc.w)
    np.testing.assert_allclose(z, z_ref, rtol=rtol, atol=atol)
    np.testing.assert_allclose(out, out_ref, rtol=rtol, atol=atol)
    # the same with physical page ids handed in: bit-identical
    phys = np.where(sel >= 0, np.take_along_axis(sc.page_table[:, None, :], np.maximum(sel, 0), axis=2), -1)
    z2, out2 = gc.decode(g, sel, n_sel, sel_phys=np.ascontiguousarray(phys, np.int32))
    assert np.array_equal(z, z2) and np.array_equal(out, out2)


@pytest.mark.parametrize("name", ["g4_d128_p64", "g8_2kv_r48_p32", "tiny_f32", "ragged_permuted"])
def test_attend_standalone_and_split_partials(name):
    """basiskv_attend alone: the merged latents, and (z_out NULL) the split
    partials left in the workspace, combined here in fp64 by the layout and
    formula the header documents; both against the oracle's latents."""
    import routed_decode_attention_amd as rda
    sc = scenario(name)
    sel, n_sel, _ = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    z_ref, _ = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    g = gc.upload(sc, cache=True, W_ofT=sc.W_ofT)
    d, w = g.d, sc.w
    sel_t, nsel_t = torch.from_numpy(sel).cuda(), torch.from_numpy(n_sel).cuda()
    z = torch.full((d.batch, d.n_q_heads, d.rank_v), float("nan"), device="cuda")
    rda.basiskv_attend(d, g.cache, g.seq_lens, g.q, sel_t, nsel_t, g.ws, z)
    torch.cuda.synchronize()
    rtol, atol = gc.tol(w)
    np.testing.assert_allclose(gc.host(z).astype(np.float64), z_ref, rtol=rtol, atol=atol)

    ws = torch.full_like(g.ws, 0xFF)  # NaN everywhere the kernel does not write
    rda.basiskv_attend(d, g.cache, g.seq_lens, g.q, sel_t, nsel_t, ws, None)
    torch.cuda.synchronize()
    ns, pairs, G, R = rda.attend_splits(d), d.batch * d.n_kv_heads, w.group, w.rank_v
    raw = gc.host(ws).view(np.float32)  # partials at the start of the workspace
    acc = raw[:pairs * ns * G * R].reshape(pairs, ns, G, R).astype(np.float64)
    ml_at = (pairs * ns * G * R * 4 + 255) // 256 * 256 // 4
    ml = raw[ml_at:ml_at + pairs * ns * G * 2].reshape(pairs, ns, G, 2).astype(np.float64)
    m, l = ml[..., 0], ml[..., 1]
    M = m.max(axis=1, keepdims=True)
    wgt = np.where(np.isfinite(M), np.exp2(m - np.where(np.isfinite(M), M, 0.0)), 0.0)  # [pairs][ns][G]
    L = (wgt * l).sum(axis=1)
    A = (wgt[..., None] * acc).sum(axis=1)
    zp = np.where(L[..., None] > 0, A / np.where(L > 0, L, 1.0)[..., None], 0.0)
    zp = zp.reshape(d.batch, d.n_kv_heads * G, R)
    np.testing.assert_allclose(zp, z_ref, rtol=rtol, atol=atol)

    # merged into z: the whole workspace NaN beforehand, so a partial read
    # before it was stored shows
    ws.fill_(0xFF)
    for _ in range(2):
        z2 = torch.full((d.batch, d.n_q_heads, d.rank_v), float("nan"), device="cuda")
        rda.basiskv_attend(d, g.cache, g.seq_lens, g.q, sel_t, nsel_t, ws, z2)
        torch.cuda.synchronize()
        np.testing.assert_allclose(gc.host(z2).astype(np.float64), z_ref, rtol=rtol, atol=atol)


@pytest.mark.parametrize("name", ["g4_d128_p64", "ragged_permuted", "g8_2kv_r48_p32"])
def test_route_physical_ids(name):
    import routed_decode_attention_amd as rda
    sc = scenario(name)
    g = gc.upload(sc, cache=True)
    B, H, K = sc.batch, sc.w.n_kv_heads, sc.w.top_k
    sel = torch.full((B, H, K), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    phys = torch.full((B, H, K), -7, dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, H, g.d.max_pages_per_seq), device="cuda")
    rda.basiskv_route(g.d, g.f, g.cache, g.seq_lens, g.q, sel, n_sel, scores, sel_phys=phys)
    torch.cuda.synchronize()
    s_, p_ = gc.host(sel), gc.host(phys)
    want = np.where(s_ >= 0, np.take_along_axis(sc.page_table[:, None, :], np.maximum(s_, 0), axis=2), -1)
    assert np.array_equal(p_, want)
    # the scores-only form: the same score bits, nothing else written
    only = torch.full_like(scores, float("nan"))
    rda.basiskv_route(g.d, g.f, g.cache, g.seq_lens, g.q, None, None, only)
    torch.cuda.synchronize()
    a, b = gc.host(scores), gc.host(only)
    for r, n in enumerate(sc.lengths):
        npg = -(-int(n) // sc.w.page_size)
        assert a[r, :, :npg].tobytes() == b[r, :, :npg].tobytes()


@pytest.mark.parametrize("name", ["g4_d128_p64", "g8_2kv_r48_p32", "ragged_permuted"])
def test_decode_with_every_page_selected(name):
    w, lengths = CASES[name]
    w = w.with_(top_k=w.max_pages_per_seq)
    sc = cases.make_scenario(w, lengths=lengths)
    sel, n_sel = cases.all_pages_selection(sc.lengths, w.n_kv_heads, w.top_k, w.page_size)
    z_ref, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    g = gc.upload(sc, cache=True, W_ofT=sc.W_ofT)
    z, out = gc.decode(g, sel, n_sel)
    rtol, atol = gc.tol(w)
    np.testing.assert_allclose(z, z_ref, rtol=rtol, atol=atol)
    np.testing.assert_allclose(out, out_ref, rtol=rtol, atol=atol)


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_step_end_to_end(name):
    """GPU writer + append + route + decode against the oracle's whole step."""
    sc = scenario(name)
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    z_ref, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    g = gc.upload(sc)
    gc.write_all(g, sc, upto_last=True, chunk=1000)
    gc.append_last(g, sc)
    gs, gn, _ = gc.route(g)
    z, out = gc.decode(g, gs, gn)
    assert np.array_equal(gn, n_sel)
    for b in range(sc.batch):
        for h in range(sc.w.n_kv_heads):
            k = int(n_sel[b, h])
            npg = -(-int(sc.lengths[b]) // sc.w.page_size)
            ranked = scores[b, h, :npg].astype(np.float64).copy()
            ranked[[j for j in range(npg) if j < sc.w.sink_pages or j >= npg - sc.w.local_pages]] = np.inf
            cases.check_selection_valid(ranked, gs[b, h, :k], k, 1e-5)
    # every row's output against the oracle re-run on the GPU's own selection
    # (equal to the oracle's up to near-tie swaps)
    cases.check_outputs_on_selection(sc, gs, gn, z, out)


def test_decode_step_at_the_page_limit():
    """The decode step (selection in the attention prologue) over 8192 pages
    of 16 tokens, the most a page-table row may hold: more pages than a
    workgroup's threads request in one batch, the rest taken by its loop;
    a second row of 70000 tokens ends in a partial page."""
    import routed_decode_attention_amd as rda
    w = small("p8k", 216, batch=2, n_q_heads=4, n_kv_heads=1, head_dim=64, page_size=16, rank_v=16, rank_k=8,
              top_k=64, d_model=128, dtype=BF16, ctx=131072)
    assert w.max_pages_per_seq == 8192
    sc = cases.make_scenario(w, lengths=[131072, 70000])
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    g = gc.upload(sc, cache=True, W_ofT=sc.W_ofT)
    pos = torch.full((2,), -1, dtype=torch.int32, device="cuda")  # no append: the cache holds every token
    kn = torch.zeros((2, 1, 64), dtype=torch.bfloat16, device="cuda")
    gsel = torch.full((2, 1, 64), -7, dtype=torch.int32, device="cuda")
    gn = torch.full((2, 1), -7, dtype=torch.int32, device="cuda")
    gsc = torch.zeros((2, 1, 8192), device="cuda")
    z = torch.zeros((2, 4, 16), device="cuda")
    out = torch.zeros((2, 128), device="cuda")
    print("[page limit] decode step over 8192 pages", flush=True)
    rda.basiskv_decode_step(g.d, g.f, g.cache, pos, kn, kn, g.seq_lens, g.q, gsel, gn, gsc, g.ws, out, z_out=z)
    torch.cuda.synchronize()
    gs, gnn, gscores = gc.host(gsel), gc.host(gn), gc.host(gsc)
    assert np.array_equal(gnn, n_sel)
    for b, n in enumerate(sc.lengths):
        npg = -(-int(n) // 16)
        np.testing.assert_allclose(gscores[b, 0, :npg], scores[b, 0, :npg], rtol=1e-5,
                                   atol=1e-5 * max(1.0, float(np.abs(scores[b, 0, :npg]).max())))
        cases.check_selection_valid(scores[b, 0, :npg].astype(np.float64), gs[b, 0, :64], 64, 1e-5)
    cases.check_outputs_on_selection(sc, gs, gnn, gc.host(z), gc.host(out))


# per-query-head selection: the headline geometry, a wide group with forced
# pages, fp32 pages (the plain kernels), and a ragged permuted mix
HEAD_SELECT = ["g4_d128_p64", "g8_mean_forced", "f32_p16_g2", "ragged_permuted"]


def _head_select_scenario(name):
    w, lengths = CASES[name]
    return cases.make_scenario(w.with_(head_select=1), lengths=lengths)


def _check_unit_selections(sc, scores, n_sel, gs, gn, gscores):
    """Every unit's GPU selection a valid top-k of the oracle's scores (forced
    pages first), its count equal, its scores within the fp32 bound."""
    w = sc.w
    assert np.array_equal(gn, n_sel)
    for b, n in enumerate(sc.lengths):
        npg = -(-int(n) // w.page_size)
        for u in range(w.units):
            k = int(n_sel[b, u])
            np.testing.assert_allclose(gscores[b, u, :npg], scores[b, u, :npg], rtol=1e-5,
                                       atol=1e-5 * max(1.0, float(np.abs(scores[b, u, :npg]).max(initial=0))))
            ranked = scores[b, u, :npg].astype(np.float64).copy()
            ranked[[j for j in range(npg) if j < w.sink_pages or j >= npg - w.local_pages]] = np.inf
            cases.check_selection_valid(ranked, gs[b, u, :k], k, 1e-5)
            assert (gs[b, u, k:] == -1).all()


@pytest.mark.parametrize("name", HEAD_SELECT)
def test_head_select_route_and_decode(name):
    """Router and decode with one selection per query head against the
    oracle: every head's selection, then every row's output re-run by the
    oracle on the GPU's selections."""
    sc = _head_select_scenario(name)
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    assert sel.shape[1] == sc.w.n_q_heads
    g = gc.upload(sc, cache=True, W_ofT=sc.W_ofT)
    gs, gn, gscores = gc.route(g)
    _check_unit_selections(sc, scores, n_sel, gs, gn, gscores)
    z, out = gc.decode(g, gs, gn)
    cases.check_outputs_on_selection(sc, gs, gn, z, out)


@pytest.mark.parametrize("name", HEAD_SELECT)
def test_head_select_decode_step(name):
    """The decode step (append fused into the scoring launch, selection in
    the attention prologue, merge fused into the projection) with one
    selection per query head, against the oracle's step."""
    import routed_decode_attention_amd as rda
    sc = _head_select_scenario(name)
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    g = gc.upload(sc, W_ofT=sc.W_ofT)
    gc.write_all(g, sc, upto_last=True, chunk=1000)
    B, U, w = sc.batch, sc.w.units, sc.w
    kn = gc.dev(np.stack([sc.K[b][int(sc.lengths[b]) - 1] for b in range(B)]), w.dtype)
    vn = gc.dev(np.stack([sc.V[b][int(sc.lengths[b]) - 1] for b in range(B)]), w.dtype)
    pos = torch.from_numpy(np.asarray(sc.lengths, np.int32) - 1).cuda()
    gsel = torch.full((B, U, w.top_k), -7, dtype=torch.int32, device="cuda")
    gnn = torch.full((B, U), -7, dtype=torch.int32, device="cuda")
    gsc = torch.zeros((B, U, w.max_pages_per_seq), device="cuda")
    z = torch.zeros((B, w.n_q_heads, w.rank_v), device="cuda")
    out = torch.zeros((B, w.d_model), device="cuda")
    rda.basiskv_decode_step(g.d, g.f, g.cache, pos, kn, vn, g.seq_lens, g.q, gsel, gnn, gsc, g.ws, out, z_out=z)
    torch.cuda.synchronize()
    gs, gn = gc.host(gsel), gc.host(gnn)
    # the GPU scored its own written cache (within the writer bound of the
    # oracle's): the oracle routes that same cache
    got = gc.cache_host(g)
    compare_written(sc, got, sc.cache)
    oc = oracle.Cache(sc.d, sc.page_table)
    for k in ("K", "Z", "S", "summ"):
        getattr(oc, k)[...] = got[k]
    _, n_sel2, scores2 = oracle.route(sc.d, sc.fac, oc, sc.lengths, sc.q)
    assert np.array_equal(n_sel2, n_sel)
    _check_unit_selections(sc, scores2, n_sel2, gs, gn, gc.host(gsc))
    cases.check_outputs_on_selection(sc, gs, gn, gc.host(z), gc.host(out))


def _permuted(sc, seed):
    pt2 = synth.permute_pool(sc.page_table, sc.num_pages, seed)
    c2 = oracle.Cache(sc.d, pt2)
    for b in range(sc.page_table.shape[0]):
        for j in range(sc.page_table.shape[1]):
            p, p2 = sc.page_table[b, j], pt2[b, j]
            if p >= 0:
                c2.K[p2], c2.Z[p2], c2.S[p2], c2.summ[p2] = sc.cache.K[p], sc.cache.Z[p], \
                    sc.cache.S[p], sc.cache.summ[p]
    return pt2, c2


@pytest.mark.parametrize("name", ["g4_d128_p64", "g8_2kv_r48_p32", "tiny_f32"])
def test_page_permutation_bit_identical(name):
    sc = scenario(name)
    g1 = gc.upload(sc, cache=True, W_ofT=sc.W_ofT)
    s1 = gc.route(g1)
    o1 = gc.decode(g1, s1[0], s1[1])
    pt2, c2 = _permuted(sc, 11)
    sc.page_table, sc.cache = pt2, c2
    g2 = gc.upload(sc, cache=True, W_ofT=sc.W_ofT)
    s2 = gc.route(g2)
    o2 = gc.decode(g2, s2[0], s2[1])
    for a, b in zip(s1[:2], s2[:2]):
        assert np.array_equal(a, b)
    for a, b in zip(o1, o2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["g4_d128_p64", "g8_2kv_r48_p32", "bf16_p16", "tiny_f32"])
def test_poisoned_unused_slots(name):
    w = CASES[name][0]
    poison = np.float32(np.nan) if w.dtype == F32 else np.uint16(0x7FC0)
    clean = scenario(name)
    dirty = scenario(name, fill=poison)
    dirty.cache.summ[...] = np.where(clean.cache.summ == 0, np.nan, dirty.cache.summ)
    r = []
    for sc in (clean, dirty):
        g = gc.upload(sc, cache=True, W_ofT=clean.W_ofT)
        s = gc.route(g)
        r.append((s, gc.decode(g, s[0], s[1])))
    assert np.array_equal(r[0][0][0], r[1][0][0])
    assert np.all(np.isfinite(r[1][1][1]))
    assert np.array_equal(r[0][1][1], r[1][1][1])


def test_run_to_run_deterministic():
    sc = scenario("g8_2kv_r48_p32")
    g = gc.upload(sc, cache=True)
    a = gc.route(g)
    oa = gc.decode(g, a[0], a[1])
    for _ in range(3):
        b = gc.route(g)
        ob = gc.decode(g, b[0], b[1])
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
        assert all(np.array_equal(x, y) for x, y in zip(oa, ob))


def test_empty_and_single_token_sequences():
    w, _ = CASES["g4_d128_p64"]
    sc = cases.make_scenario(w, lengths=[0, 1, 65])
    sel, n_sel, _ = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    z_ref, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    g = gc.upload(sc, cache=True, W_ofT=sc.W_ofT)
    gs, gn, _ = gc.route(g)
    assert gn.tolist() == [[0], [1], [2]]
    assert (gs[0] == -1).all()
    z, out = gc.decode(g, gs, gn)
    assert (out[0] == 0).all() and (z[0] == 0).all()
    np.testing.assert_allclose(out, out_ref, rtol=2e-2, atol=2e-3)


def test_decode_step_edge_rows():
    """The decode step (append fused into the router's cluster) over rows that
    are empty, hold one token, start a page, append past the last page
    (skipped), or append nothing (pos -1): against the oracle on the cache
    those appends produce."""
    import routed_decode_attention_amd as rda
    w, _ = CASES["g4_d128_p64"]
    lengths = [0, 1, 65, 700, 300]
    pos = np.array([-1, 0, 64, 699, -1], np.int32)
    cap = w.max_pages_per_seq * w.page_size
    sc = cases.make_scenario(w.with_(batch=len(lengths)), lengths=lengths)  # the oracle cache holds every token
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    z_ref, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    g = gc.upload(sc, W_ofT=sc.W_ofT)
    for b, n in enumerate(lengths):  # what the cache holds before the step
        m = n - 1 if pos[b] >= 0 else n
        if m > 0:
            rda.basiskv_write(g.d, g.f, g.cache, b, 0, gc.dev(sc.K[b][:m], w.dtype), gc.dev(sc.V[b][:m], w.dtype))
    B = len(lengths)
    last = lambda X, b: X[b][max(lengths[b] - 1, 0)] if lengths[b] else np.zeros_like(sc.K[3][0])
    kn = gc.dev(np.stack([last(sc.K, b) for b in range(B)]), w.dtype)
    vn = gc.dev(np.stack([last(sc.V, b) for b in range(B)]), w.dtype)
    pos_d = torch.from_numpy(pos).cuda()
    pos_d[4] = cap  # past the last page: skipped like -1
    gsel = torch.full((B, 1, w.top_k), -7, dtype=torch.int32, device="cuda")
    gn = torch.full((B, 1), -7, dtype=torch.int32, device="cuda")
    gscores = torch.zeros((B, 1, w.max_pages_per_seq), device="cuda")
    z = torch.zeros((B, w.n_q_heads, w.rank_v), device="cuda")
    out = torch.zeros((B, w.d_model), device="cuda")
    rda.basiskv_decode_step(g.d, g.f, g.cache, pos_d, kn, vn, g.seq_lens, g.q, gsel, gn, gscores, g.ws, out,
                            z_out=z)
    torch.cuda.synchronize()
    gs, gnn = gc.host(gsel), gc.host(gn)
    assert np.array_equal(gnn, n_sel)
    assert (gs[0] == -1).all() and (gc.host(out)[0] == 0).all()
    for b, n in enumerate(lengths):
        npg = -(-n // w.page_size)
        k = int(n_sel[b, 0])
        cases.check_selection_valid(scores[b, 0, :npg], gs[b, 0, :k], k, 1e-5)
    cases.check_outputs_on_selection(sc, gs, gnn, gc.host(z), gc.host(out))


@pytest.mark.parametrize("name,chunks", [("g4_d128_p64", [0, 128, 300]), ("g8_2kv_r48_p32", [0, 77, 513]),
                                         ("tiny_f32", [0, 64, 200]), ("bf16_p16", [0, 40, 100])])
def test_prefill_matches_oracle(name, chunks):
    w, _ = CASES[name]
    n = chunks[-1]
    w = w.with_(batch=1)
    sc = cases.make_scenario(w, lengths=[n], write=False)
    qp = synth.to_storage(np.random.default_rng(5).standard_normal((n, w.n_q_heads, w.head_dim)), w.dtype)
    ora = oracle.Cache(sc.d, sc.page_table)
    W = oracle.fold(sc.d, sc.fac.B, sc.fac.W_O)
    zr, orr = [], []
    for a, b in zip(chunks[:-1], chunks[1:]):
        z, o = oracle.prefill(sc.d, sc.fac, W, ora, 0, a, qp[a:b], sc.K[0][a:b], sc.V[0][a:b])
        zr.append(z); orr.append(o)
    z_ref, out_ref = np.concatenate(zr), np.concatenate(orr)
    g = gc.upload(sc, W_ofT=W, max_prefill=n)
    zs, outs = [], []
    for a, b in zip(chunks[:-1], chunks[1:]):
        z = torch.empty((b - a, w.n_q_heads, w.rank_v), device="cuda")
        out = torch.empty((b - a, w.d_model), device="cuda")
        import routed_decode_attention_amd as rda
        rda.basiskv_prefill(g.d, g.f, g.cache, 0, a, gc.dev(qp[a:b], w.dtype), gc.dev(sc.K[0][a:b], w.dtype),
                            gc.dev(sc.V[0][a:b], w.dtype), g.ws, out, z_out=z)
        zs.append(gc.host(z)); outs.append(gc.host(out))
    torch.cuda.synchronize()
    rtol, atol = gc.tol(w)
    np.testing.assert_allclose(np.concatenate(zs), z_ref, rtol=rtol, atol=atol)
    np.testing.assert_allclose(np.concatenate(outs), out_ref, rtol=rtol, atol=atol)
    compare_written(sc, gc.cache_host(g), ora)


@pytest.mark.parametrize("split_pages", [1, 3])
def test_prefill_key_range_splits(split_pages, monkeypatch):
    """Prefill chunks whose key pages are split into many ranges (split_pages
    pages each, at most eight ranges; ranges past a row block's last page are
    empty and leave empty partials): against the oracle, as unsplit."""
    monkeypatch.setenv("BASISKV_PREFILL_SPLIT_PAGES", str(split_pages))
    print(f"[prefill splits] {split_pages} pages a range", flush=True)
    test_prefill_matches_oracle("g8_2kv_r48_p32", [0, 77, 513])   # 17 pages of 32
    test_prefill_matches_oracle("g4_d128_p64", [0, 128, 300])     # 5 pages of 64


@pytest.mark.parametrize("rows,nq,r,dm", [(65, 2, 48, 256), (300, 4, 32, 512), (2048, 8, 48, 4096)])
def test_project_many_rows(rows, nq, r, dm):
    """The projection over many rows (the prefill chunks' LDS-staged 128 x 256
    tiles) against the fp64 product of the same bf16 weights: rows past a
    tile's end, a contraction of an odd number of 32-wide steps (96), the
    8K prefill's chunk shape.  z enters as bf16 high + low parts (about 16
    significant bits), so the product is within a few 1e-5 of the exact one."""
    import routed_decode_attention_amd as rda
    rng = np.random.default_rng(rows + dm)
    kdim = nq * r
    d = rda.Dims(batch=1, n_q_heads=nq, n_kv_heads=1, head_dim=128, rank_v=r, rank_k=16, page_size=64,
                 d_model=dm, top_k=1, max_pages_per_seq=1, num_phys_pages=1, dtype=BF16)
    W = synth.to_storage(rng.standard_normal((dm, kdim)) / np.sqrt(kdim), BF16)  # bf16 bits
    z = rng.standard_normal((rows, kdim)).astype(np.float32)
    f = rda.Factors(B=torch.zeros(128 * r, device="cuda"), P=torch.zeros(r * 128, device="cuda"),
                    R_enc=torch.zeros(128 * 16, device="cuda"), R_dec=torch.zeros(16 * 128, device="cuda"),
                    W_ofT=gc.dev(W, BF16))
    out = torch.full((rows, dm), float("nan"), device="cuda")
    print(f"[project] rows {rows} kdim {kdim} d_model {dm}", flush=True)
    rda.basiskv_project(d, f, torch.from_numpy(z).cuda(), rows, out)
    torch.cuda.synchronize()
    Wf = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = z.astype(np.float64) @ Wf.T
    got = gc.host(out)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-3, atol=1e-4 * np.abs(ref).max())


def test_prefill_interleaved_with_decode_steps():
    """Serving order: sequence 0 is prefilled chunk by chunk while the other
    rows run decode steps (row 0 inactive: length 0, no append) between the
    chunks; then row 0 joins a decode step over its prefilled cache.  Every
    chunk and every step against the oracle run in the same order on its own
    cache, and the final caches against each other."""
    import routed_decode_attention_amd as rda
    w, _ = CASES["g4_d128_p64"]
    final = [450, 300, 129, 64]
    chunks = [0, 150, 300, 450]
    B, steps = len(final), len(chunks) - 1
    w = w.with_(batch=B)
    sc = cases.make_scenario(w, lengths=final, write=False)
    qp = synth.to_storage(np.random.default_rng(11).standard_normal((final[0], w.n_q_heads, w.head_dim)), w.dtype)
    ora = oracle.Cache(sc.d, sc.page_table)
    W = oracle.fold(sc.d, sc.fac.B, sc.fac.W_O)
    g = gc.upload(sc, W_ofT=W, max_prefill=final[0])
    for b in range(1, B):  # the decoding rows hold all but their last `steps` tokens
        m = final[b] - steps
        oracle.write(sc.d, sc.fac, ora, b, 0, sc.K[b][:m], sc.V[b][:m])
        rda.basiskv_write(g.d, g.f, g.cache, b, 0, gc.dev(sc.K[b][:m], w.dtype), gc.dev(sc.V[b][:m], w.dtype))
    rtol, atol = gc.tol(w)

    def decode_step(lengths, pos):
        """One decode step on both sides; rows with pos >= 0 append token pos."""
        for b in range(B):
            if pos[b] >= 0:
                oracle.write(sc.d, sc.fac, ora, b, int(pos[b]), sc.K[b][pos[b]:pos[b] + 1],
                             sc.V[b][pos[b]:pos[b] + 1])
        lens = np.asarray(lengths, np.int32)
        sel, n_sel, scores = oracle.route(sc.d, sc.fac, ora, lens, sc.q)
        _, out_ref = oracle.decode(sc.d, W, ora, lens, sc.q, sel, n_sel)
        tok = lambda X, b: X[b][max(int(pos[b]), 0)]
        kn = gc.dev(np.stack([tok(sc.K, b)[None] for b in range(B)]), w.dtype)
        vn = gc.dev(np.stack([tok(sc.V, b)[None] for b in range(B)]), w.dtype)
        g.seq_lens.copy_(torch.from_numpy(lens))
        gsel = torch.full((B, 1, w.top_k), -7, dtype=torch.int32, device="cuda")
        gn = torch.full((B, 1), -7, dtype=torch.int32, device="cuda")
        gscores = torch.zeros((B, 1, w.max_pages_per_seq), device="cuda")
        out = torch.zeros((B, w.d_model), device="cuda")
        rda.basiskv_decode_step(g.d, g.f, g.cache, torch.from_numpy(np.asarray(pos, np.int32)).cuda(), kn, vn,
                                g.seq_lens, g.q, gsel, gn, gscores, g.ws, out)
        torch.cuda.synchronize()
        gs, gnn, go = gc.host(gsel), gc.host(gn), gc.host(out)
        assert np.array_equal(gnn, n_sel)
        for b in range(B):
            k = int(n_sel[b, 0])
            if lengths[b] == 0:
                assert k == 0 and (go[b] == 0).all()
                continue
            npg = -(-int(lengths[b]) // w.page_size)
            cases.check_selection_valid(scores[b, 0, :npg], gs[b, 0, :k], k, 1e-5)
        # every row against the oracle re-run on the GPU's selection
        _, out_gsel = oracle.decode(sc.d, W, ora, lens, sc.q, gs, gnn)
        np.testing.assert_allclose(go, out_gsel, rtol=2e-2, atol=2e-3)

    for i in range(steps):
        a, e = chunks[i], chunks[i + 1]
        z_ref, o_ref = oracle.prefill(sc.d, sc.fac, W, ora, 0, a, qp[a:e], sc.K[0][a:e], sc.V[0][a:e])
        z = torch.empty((e - a, w.n_q_heads, w.rank_v), device="cuda")
        out = torch.empty((e - a, w.d_model), device="cuda")
        rda.basiskv_prefill(g.d, g.f, g.cache, 0, a, gc.dev(qp[a:e], w.dtype), gc.dev(sc.K[0][a:e], w.dtype),
                            gc.dev(sc.V[0][a:e], w.dtype), g.ws, out, z_out=z)
        torch.cuda.synchronize()
        np.testing.assert_allclose(gc.host(z), z_ref, rtol=rtol, atol=atol)
        np.testing.assert_allclose(gc.host(out), o_ref, rtol=rtol, atol=atol)
        p = [-1] + [final[b] - steps + i for b in range(1, B)]
        decode_step([0] + [final[b] - steps + i + 1 for b in range(1, B)], p)
    decode_step(final, [-1] * B)  # row 0 joins: routed attention over its prefilled pages
    compare_written(sc, gc.cache_host(g), ora)


@pytest.mark.parametrize("pages_per_wg", [None, 5, 256])
@pytest.mark.parametrize("name", ["g4_d128_p64", "g8_2kv_r48_p32", "ragged_permuted", "tiny_f32", "g4_forced",
                                  "g8_mean_forced"])
def test_fused_append_route_equals_separate_calls(name, pages_per_wg, monkeypatch):
    """The decode step (the append fused with the scores; the selection in
    the attention kernel's prologue; with pages_per_wg set, scoring
    workgroups of that many pages) against separate append, route and
    decode calls: bit-identical."""
    import routed_decode_attention_amd as rda
    if pages_per_wg is not None:
        monkeypatch.setenv("BASISKV_SCORE_PAGES_PER_WG", str(pages_per_wg))
    sc = scenario(name)
    outs = []
    for fused in (False, True):
        g = gc.upload(sc)
        gc.write_all(g, sc, upto_last=True, chunk=333)
        B = sc.batch
        kn = gc.dev(np.stack([sc.K[b][int(sc.lengths[b]) - 1] for b in range(B)]), sc.w.dtype)
        vn = gc.dev(np.stack([sc.V[b][int(sc.lengths[b]) - 1] for b in range(B)]), sc.w.dtype)
        pos = torch.from_numpy(np.asarray(sc.lengths, np.int32) - 1).cuda()
        sel = torch.full((B, g.d.n_kv_heads, g.d.top_k), -7, dtype=torch.int32, device="cuda")
        n_sel = torch.zeros((B, g.d.n_kv_heads), dtype=torch.int32, device="cuda")
        scores = torch.zeros((B, g.d.n_kv_heads, g.d.max_pages_per_seq), device="cuda")
        z = torch.zeros((B, g.d.n_q_heads, g.d.rank_v), device="cuda")
        out = torch.zeros((B, g.d.d_model), device="cuda")
        if fused:
            rda.basiskv_decode_step(g.d, g.f, g.cache, pos, kn, vn, g.seq_lens, g.q, sel, n_sel, scores,
                                    g.ws, out, z_out=z)
        else:
            rda.basiskv_append(g.d, g.f, g.cache, pos, kn, vn)
            rda.basiskv_route(g.d, g.f, g.cache, g.seq_lens, g.q, sel, n_sel, scores)
            rda.basiskv_decode(g.d, g.f, g.cache, g.seq_lens, g.q, sel, n_sel, g.ws, out, z_out=z)
        torch.cuda.synchronize()
        npg = [-(-int(n) // sc.w.page_size) for n in sc.lengths]
        sc_host = gc.host(scores)
        outs.append((gc.cache_host(g), gc.host(sel), gc.host(n_sel),
                     [sc_host[b, :, :npg[b]] for b in range(B)], gc.host(out), gc.host(z)))
    a, b = outs
    for k in a[0]:
        assert np.array_equal(a[0][k], b[0][k]), k
    for x, y in zip(a[1:3] + a[4:], b[1:3] + b[4:]):
        assert np.array_equal(x, y)
    for x, y in zip(a[3], b[3]):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("ppw,waves", [(1, 4), (2, 4), (3, 8), (5, 8), (1, 8)])
def test_pages_per_wave_plans(ppw, waves, monkeypatch):
    """Every split plan (4 or 8 waves per workgroup; one page per wave, or
    several with the next page's loads overlapping) matches the oracle; the
    ragged tail of the selection lands in a partly filled wave."""
    monkeypatch.setenv("BASISKV_PAGES_PER_WAVE", str(ppw))
    monkeypatch.setenv("BASISKV_ATTEND_WAVES", str(waves))
    for name in ("g4_d128_p64", "g8_2kv_r48_p32"):
        w, lengths = CASES[name]
        w = w.with_(top_k=11)
        sc = cases.make_scenario(w, lengths=lengths)
        sel, n_sel, _ = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
        z_ref, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
        g = gc.upload(sc, cache=True, W_ofT=sc.W_ofT)
        z, out = gc.decode(g, sel, n_sel)
        np.testing.assert_allclose(z, z_ref, rtol=2e-2, atol=2e-3)
        np.testing.assert_allclose(out, out_ref, rtol=2e-2, atol=2e-3)
