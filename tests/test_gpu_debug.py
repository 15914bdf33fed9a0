"""Debug mode (BASISKV_DEBUG=1): calls check the device data they are about
to read and return BASISKV_E_DATA, with nothing else enqueued, on a
violation; on valid data the results are those of release mode.

The planted values stay inside the allocations: the pools carry spare pages
past num_phys_pages, the selection spare rows, so that even an unchecked
read could not leave device memory."""
import numpy as np
import pytest
import torch

from tests import cases, gpu_cases as gc
from workloads import configs

pytestmark = pytest.mark.gpu
SPARE = 8  # pool pages past num_phys_pages


def _scenario():
    w = configs.get("llama8b_32k").with_(name="dbg", cfg_id=301, batch=3, top_k=5, d_model=256)
    return cases.make_scenario(w, lengths=[700, 64, 130])


def _padded(g):
    """The device pools with SPARE zero pages past the declared pool."""
    import routed_decode_attention_amd as rda
    c = g.cache
    pad = lambda t: torch.cat([t, torch.zeros((SPARE,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)])
    g.cache = rda.Cache(K=pad(c.K), Z=pad(c.Z), S=pad(c.S), summ=pad(c.summ), page_table=c.page_table.clone())
    return g


def _step(g, sc, sel, n_sel):
    import routed_decode_attention_amd as rda
    B = sc.batch
    kn = gc.dev(np.stack([sc.K[b][int(sc.lengths[b]) - 1] for b in range(B)]), sc.w.dtype)
    vn = gc.dev(np.stack([sc.V[b][int(sc.lengths[b]) - 1] for b in range(B)]), sc.w.dtype)
    pos = torch.from_numpy(np.asarray(sc.lengths, np.int32) - 1).cuda()
    scores = torch.zeros((B, g.d.n_kv_heads, g.d.max_pages_per_seq), device="cuda")
    out = torch.zeros((B, g.d.d_model), device="cuda")
    rda.basiskv_decode_step(g.d, g.f, g.cache, pos, kn, vn, g.seq_lens, g.q, sel, n_sel, scores, g.ws, out)
    torch.cuda.synchronize()
    return gc.host(out)


def test_valid_data_gives_release_results(monkeypatch):
    sc = _scenario()
    outs = []
    for debug in ("0", "1"):
        monkeypatch.setenv("BASISKV_DEBUG", debug)
        g = _padded(gc.upload(sc))
        gc.write_all(g, sc, upto_last=True, chunk=300)
        sel = torch.zeros((sc.batch, 1, g.d.top_k), dtype=torch.int32, device="cuda")
        n_sel = torch.zeros((sc.batch, 1), dtype=torch.int32, device="cuda")
        outs.append((_step(g, sc, sel, n_sel), gc.host(sel), gc.cache_host(g)))
    a, b = outs
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for k in a[2]:
        assert np.array_equal(a[2][k], b[2][k]), k


def test_bad_page_table_entries_and_lengths(monkeypatch):
    import routed_decode_attention_amd as rda
    monkeypatch.setenv("BASISKV_DEBUG", "1")
    sc = _scenario()
    g = _padded(gc.upload(sc, cache=True, W_ofT=sc.W_ofT))
    nphys = g.d.num_phys_pages
    good_pt = g.cache.page_table.clone()

    def expect_data_error(fn, what):
        with pytest.raises(rda.BasisKVError) as e:
            fn()
        assert e.value.code == rda.E_DATA, (what, str(e.value))
        return str(e.value)

    sel = torch.full((sc.batch, 1, g.d.top_k), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((sc.batch, 1), -7, dtype=torch.int32, device="cuda")
    scores = torch.zeros((sc.batch, 1, g.d.max_pages_per_seq), device="cuda")
    # a page of row 0 inside its length maps past the pool
    g.cache.page_table[0, 3] = nphys + 3
    msg = expect_data_error(lambda: rda.basiskv_route(g.d, g.f, g.cache, g.seq_lens, g.q, sel, n_sel, scores),
                            "route")
    assert "page-table entry" in msg
    torch.cuda.synchronize()
    assert (gc.host(sel) == -7).all() and (gc.host(n_sel) == -7).all()  # nothing ran
    expect_data_error(lambda: _step(g, sc, sel, n_sel), "decode_step")
    kv = gc.dev(sc.K[0][:10], sc.w.dtype)
    expect_data_error(lambda: rda.basiskv_write(g.d, g.f, g.cache, 0, 200, kv, kv), "write")  # page 3
    q1 = gc.dev(np.zeros((10, g.d.n_q_heads, g.d.head_dim), np.uint16), sc.w.dtype)  # bf16 bits
    ws = rda.new_workspace(g.d, 10)
    out = torch.zeros((10, g.d.d_model), device="cuda")
    expect_data_error(lambda: rda.basiskv_prefill(g.d, g.f, g.cache, 0, 300, q1, kv, kv, ws, out), "prefill")
    # the page of an append position
    g.cache.page_table.copy_(good_pt)
    g.cache.page_table[1, 0] = nphys + 1
    pos = torch.tensor([5, 10, 20], dtype=torch.int32, device="cuda")
    kn = gc.dev(np.zeros((3, 1, g.d.head_dim), np.uint16), sc.w.dtype)  # bf16 bits
    msg = expect_data_error(lambda: rda.basiskv_append(g.d, g.f, g.cache, pos, kn, kn), "append")
    assert "append position" in msg
    # a length past max_pages_per_seq * page_size
    g.cache.page_table.copy_(good_pt)
    g.seq_lens[2] = g.d.max_pages_per_seq * g.d.page_size + 1
    msg = expect_data_error(lambda: rda.basiskv_route(g.d, g.f, g.cache, g.seq_lens, g.q, sel, n_sel, scores),
                            "route length")
    assert "sequence length" in msg


def test_bad_selections(monkeypatch):
    import routed_decode_attention_amd as rda
    monkeypatch.setenv("BASISKV_DEBUG", "1")
    sc = _scenario()
    g = _padded(gc.upload(sc, cache=True, W_ofT=sc.W_ofT))
    s, n, _ = gc.route(g)
    B, K = sc.batch, g.d.top_k
    npg = [-(-int(x) // g.d.page_size) for x in sc.lengths]
    # spare rows past the selection, in case an unchecked read ran on
    sel_big = torch.zeros((B + 1, 1, K), dtype=torch.int32, device="cuda")
    z = torch.zeros((B, g.d.n_q_heads, g.d.rank_v), device="cuda")

    def attend(sel_np, n_np, phys=None):
        sel_big[:B] = torch.from_numpy(sel_np).cuda()
        rda.basiskv_attend(g.d, g.cache, g.seq_lens, g.q, sel_big[:B], torch.from_numpy(n_np).cuda(), g.ws,
                           z, sel_phys=phys)
        torch.cuda.synchronize()

    attend(s, n)  # the router's own selection passes
    bad_count = n.copy()
    bad_count[0, 0] = K + 1
    with pytest.raises(rda.BasisKVError) as e:
        attend(s, bad_count)
    assert e.value.code == rda.E_DATA
    # row 1 has npg[1] pages: page npg[1] is past its end (still below
    # max_pages, and mapped here so that an unchecked read stays in the pool)
    g.cache.page_table[1, npg[1]] = 0
    bad_page = s.copy()
    bad_page[1, 0, 0] = npg[1]
    with pytest.raises(rda.BasisKVError) as e:
        attend(bad_page, n)
    assert e.value.code == rda.E_DATA
    phys = torch.from_numpy(np.where(s >= 0, sc.page_table[np.arange(B)[:, None, None], np.maximum(s, 0)], -1)
                            .astype(np.int32)).cuda()
    attend(s, n, phys)
    phys[0, 0, 0] = g.d.num_phys_pages + 2
    with pytest.raises(rda.BasisKVError) as e:
        attend(s, n, phys)
    assert e.value.code == rda.E_DATA


def test_checks_from_two_host_threads_do_not_cross(monkeypatch):
    """Two host threads on their own streams, one with valid lengths and one
    with a length past the cache, call the router in debug mode together:
    every valid call succeeds and every invalid one returns BASISKV_E_DATA."""
    import threading
    import routed_decode_attention_amd as rda
    monkeypatch.setenv("BASISKV_DEBUG", "1")
    sc = _scenario()
    g = _padded(gc.upload(sc, cache=True, W_ofT=sc.W_ofT))
    bad = g.seq_lens.clone()
    bad[2] = g.d.max_pages_per_seq * g.d.page_size + 1
    torch.cuda.synchronize()
    results = {"good": [], "bad": []}

    def run(kind, lens):
        st = torch.cuda.Stream()
        sel = torch.zeros((sc.batch, 1, g.d.top_k), dtype=torch.int32, device="cuda")
        n_sel = torch.zeros((sc.batch, 1), dtype=torch.int32, device="cuda")
        scores = torch.zeros((sc.batch, 1, g.d.max_pages_per_seq), device="cuda")
        torch.cuda.synchronize()
        for _ in range(40):
            try:
                rda.basiskv_route(g.d, g.f, g.cache, lens, g.q, sel, n_sel, scores, stream=st)
                results[kind].append(0)
            except rda.BasisKVError as e:
                results[kind].append(e.code)
        st.synchronize()

    threads = [threading.Thread(target=run, args=("good", g.seq_lens)), threading.Thread(target=run, args=("bad", bad))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert results["good"] == [0] * 40, results["good"]
    assert results["bad"] == [rda.E_DATA] * 40, results["bad"]
