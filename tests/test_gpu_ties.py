"""GPU router on exact score ties: selections bit-equal to the oracle's.

The cases (tests/tie_constructions.py) make pages share their score bits on
both sides, so only the tie rule decides what is kept: larger score first,
then the smaller logical page (weekinpapers "BasisKV: Value Latents for
Communication and Key Routing", Abstract: the router identifies which Key
pages are read).  Shapes with at most 512 pages and 2 <= top_k <= 64, with
top_k above 64 and with more than 512 pages are covered; the selection runs
in the selection kernel (route, append + route) and in the attention
kernel's prologue (the decode step), under two scoring plans, and with the
decode-step append whose new page ties a kept page.

Scores of exactly zero cannot carry a sign here: every GPU score is an fma
chain started from +0, so -0 never reaches the selection; the oracle's
-0 == +0 rule is pinned on the CPU (tests/test_oracle_pins.py).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import tie_constructions as tk

pytestmark = pytest.mark.gpu

gc = None


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    global gc
    assert torch.cuda.is_available(), "GPU tie tests need a GPU"
    from tests import gpu_cases
    gc = gpu_cases
    oracle.build(force=False)


@pytest.mark.parametrize("pages_per_wg", [None, 7])
@pytest.mark.parametrize("name", [s[0] for s in tk.SUMMARY_SHAPES])
def test_route_ties_bit_equal(name, pages_per_wg, monkeypatch):
    sc, k, tied = tk.summary_case(name)
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    g = gc.upload(sc, cache=True)
    if pages_per_wg is None:
        gs, gn, gsc = gc.route(g)
    else:
        monkeypatch.setenv("BASISKV_SCORE_PAGES_PER_WG", str(pages_per_wg))
        gs, gn, gsc = gc.route(g)
    print(f"[ties] {name} pages_per_wg={pages_per_wg}", flush=True)
    assert np.array_equal(gn, n_sel)
    assert np.array_equal(gs, sel), [(b, gs[b, 0, :k].tolist(), sel[b, 0, :k].tolist()) for b in range(sc.batch)
                                     if not np.array_equal(gs[b], sel[b])]
    for b in range(sc.batch):
        assert len({gsc[b, 0, j].tobytes() for j in tied[b]}) <= 1, "tied pages share their GPU score bits"


def _append_inputs(sc):
    n = int(sc.lengths[0])
    kn = gc.dev(sc.K[0][n - 1:n], sc.w.dtype)
    vn = gc.dev(sc.V[0][n - 1:n], sc.w.dtype)
    pos = torch.tensor([n - 1], dtype=torch.int32, device="cuda")
    return kn, vn, pos


@pytest.mark.parametrize("mode", ["fused_single", "fused_cluster", "decode_step"])  # fused_*: append_route
@pytest.mark.parametrize("name", [s[0] for s in tk.APPEND_SHAPES])
def test_appended_page_ties_bit_equal(name, mode, monkeypatch):
    """The decode-step append fills the last page with a copy of the page at
    the selection boundary: the appended page must lose the tie (side 0) or
    be kept beside it (side 1), exactly as the oracle decides."""
    import routed_decode_attention_amd as rda
    sc, k, src, side = tk.append_case(name)
    sel, n_sel, _ = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    z_ref, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, n_sel)
    g = gc.upload(sc, W_ofT=sc.W_ofT)
    gc.write_all(g, sc, upto_last=True, chunk=1000)
    kn, vn, pos = _append_inputs(sc)
    d = g.d
    gsel = torch.full((1, 1, k), -7, dtype=torch.int32, device="cuda")
    gn = torch.full((1, 1), -7, dtype=torch.int32, device="cuda")
    gscores = torch.zeros((1, 1, d.max_pages_per_seq), device="cuda")
    print(f"[ties] {name} {mode}", flush=True)
    if mode == "fused_single":
        rda.basiskv_append_route(d, g.f, g.cache, pos, kn, vn, g.seq_lens, g.q, gsel, gn, gscores)
    elif mode == "fused_cluster":
        monkeypatch.setenv("BASISKV_SCORE_PAGES_PER_WG", "13")
        rda.basiskv_append_route(d, g.f, g.cache, pos, kn, vn, g.seq_lens, g.q, gsel, gn, gscores)
    else:
        out = torch.zeros((1, d.d_model), device="cuda")
        z = torch.zeros((1, d.n_q_heads, d.rank_v), device="cuda")
        rda.basiskv_decode_step(d, g.f, g.cache, pos, kn, vn, g.seq_lens, g.q, gsel, gn, gscores, g.ws, out,
                                z_out=z)
    torch.cuda.synchronize()
    gs, gnn, gsc = gc.host(gsel), gc.host(gn), gc.host(gscores)
    npg = int(sc.lengths[0]) // sc.w.page_size
    assert gsc[0, 0, src].tobytes() == gsc[0, 0, npg - 1].tobytes(), "the copied page ties on the GPU"
    assert np.array_equal(gnn, n_sel)
    assert np.array_equal(gs, sel), (gs[0, 0].tolist(), sel[0, 0].tolist())
    if mode == "decode_step":
        np.testing.assert_allclose(gc.host(out).astype(np.float64), out_ref, rtol=2e-2, atol=2e-3)
        np.testing.assert_allclose(gc.host(z).astype(np.float64), z_ref, rtol=2e-2, atol=2e-3)
