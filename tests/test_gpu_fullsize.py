"""Full-size parity: the workloads at their real shapes, through the same
entry points and launch plans the benchmark times.

The GPU writes every sequence's cache with its own writer and runs the decode
step (append + route + attend + project) over the whole batch.  The oracle
rebuilds only a few sampled sequences from the same seeded inputs (its own
writer, its own cache).  Checks, on the sampled rows:
  1. the GPU-written pages against the oracle's writer (Keys bit for bit,
     latents/residuals within the fp32 accumulation bound plus one bf16 ulp,
     page sums = the slot-order sum of the stored values);
  2. with those rows' pages then overwritten by the oracle's (identical cache
     contents), the GPU route + decode over the whole batch: selected sets
     identical up to swaps of pages whose oracle scores differ by < 1e-5
     relative, scores within 1e-5, outputs within rtol 2e-2 / atol 2e-3;
  3. the end-to-end output of step 1's cache, where its selection equals the
     oracle's.
The 8192-token prefill is compared on sampled query rows of every chunk.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import cases
from workloads import configs, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gc():
    assert torch.cuda.is_available(), "full-size parity needs a GPU"
    from tests import gpu_cases
    oracle.build(force=False)
    return gpu_cases


def _decode_full(gc, name, sample):
    print(f"[fullsize] {name}: rows {sample}", flush=True)
    import routed_decode_attention_amd as rda
    w = configs.get(name)
    B, H = w.batch, w.n_kv_heads
    fac = synth.make_factors(w)
    lengths = synth.make_lengths(w)
    pt, total = synth.make_page_table(w, lengths)
    d = gc.dims_of(w, B, total)
    f = rda.Factors(B=gc.dev(fac.B, 0), P=gc.dev(fac.P, 0), R_enc=gc.dev(fac.R_enc, 0),
                    R_dec=gc.dev(fac.R_dec, 0))
    f.W_ofT = torch.empty((w.d_model, w.n_q_heads * w.rank_v), dtype=d.torch_dtype, device="cuda")
    rda.basiskv_fold_output(d, f.B, gc.dev(fac.W_O, w.dtype), f.W_ofT)
    cache = rda.Cache.empty(d, torch.from_numpy(pt))
    kn, vn = [], []
    for b in range(B):
        n = int(lengths[b])
        K, V = synth.make_sequence(w, fac, b, n)
        rda.basiskv_write(d, f, cache, b, 0, gc.dev(K[:n - 1], w.dtype), gc.dev(V[:n - 1], w.dtype))
        kn.append(K[n - 1])
        vn.append(V[n - 1])
        del K, V
    seq_lens = torch.from_numpy(lengths.astype(np.int32)).cuda()
    pos = (seq_lens - 1).contiguous()
    q = gc.dev(synth.make_queries(w), w.dtype)
    ws = rda.new_workspace(d)
    sel = torch.zeros((B, H, w.top_k), dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, H, w.max_pages_per_seq), device="cuda")
    z = torch.zeros((B, w.n_q_heads, w.rank_v), device="cuda")
    out = torch.zeros((B, w.d_model), device="cuda")
    rda.basiskv_decode_step(d, f, cache, pos, gc.dev(np.stack(kn), w.dtype), gc.dev(np.stack(vn), w.dtype),
                            seq_lens, q, sel, n_sel, scores, ws, out, z_out=z)
    torch.cuda.synchronize()
    e2e_sel, e2e_nsel, e2e_out = gc.host(sel), gc.host(n_sel), gc.host(out).astype(np.float64)

    # the oracle on the sampled sequences only (its own placement of their pages)
    sc = cases.make_scenario(w, rows=sample)
    o_sel, o_nsel, o_scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    z_ref, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, o_sel, o_nsel)

    # 1. the GPU writer on the sampled rows
    gpt = pt[sample]
    cases.compare_written(sc, gc.cache_host(gc.Dev(w, d, f, cache, seq_lens, q, ws)), sc.cache,
                          got_page_table=gpt)

    # 2. identical cache contents on the sampled rows, then route + decode of the batch
    src, dst = [], []
    for i, b in enumerate(sample):
        npg = -(-int(lengths[b]) // w.page_size)
        src += sc.page_table[i, :npg].tolist()
        dst += pt[b, :npg].tolist()
    src, dst = np.array(src), torch.from_numpy(np.array(dst)).cuda()
    cache.K[dst] = gc.dev(sc.cache.K[src], w.dtype)
    cache.Z[dst] = gc.dev(sc.cache.Z[src], w.dtype)
    cache.S[dst] = gc.dev(sc.cache.S[src], w.dtype)
    cache.summ[dst] = gc.dev(sc.cache.summ[src], 0)
    rda.basiskv_route(d, f, cache, seq_lens, q, sel, n_sel, scores)
    torch.cuda.synchronize()
    g_sel, g_nsel, g_scores = gc.host(sel), gc.host(n_sel), gc.host(scores)
    import os
    os.environ["BASISKV_SCORE_PAGES_PER_WG"] = "256"  # another scoring plan: same bits
    try:
        rda.basiskv_route(d, f, cache, seq_lens, q, sel, n_sel, scores)
    finally:
        del os.environ["BASISKV_SCORE_PAGES_PER_WG"]
    torch.cuda.synchronize()
    assert np.array_equal(gc.host(sel), g_sel) and np.array_equal(gc.host(n_sel), g_nsel)
    for i, b in enumerate(sample):
        npg = -(-int(lengths[b]) // w.page_size)
        for g in range(H):
            k = int(o_nsel[i, g])
            assert int(g_nsel[b, g]) == k
            np.testing.assert_allclose(g_scores[b, g, :npg], o_scores[i, g, :npg], rtol=1e-5,
                                       atol=1e-5 * max(1.0, float(np.abs(o_scores[i, g, :npg]).max())))
            cases.check_selection_valid(o_scores[i, g, :npg], g_sel[b, g, :k], k, 1e-5)
    # the GPU decode over the oracle's selection on the sampled rows
    sel_mix, nsel_mix = g_sel.copy(), g_nsel.copy()
    for i, b in enumerate(sample):
        sel_mix[b], nsel_mix[b] = o_sel[i], o_nsel[i]
    rda.basiskv_decode(d, f, cache, seq_lens, q, torch.from_numpy(sel_mix).cuda(),
                       torch.from_numpy(nsel_mix).cuda(), ws, out, z_out=z)
    torch.cuda.synchronize()
    got, got_z = gc.host(out).astype(np.float64), gc.host(z).astype(np.float64)
    for i, b in enumerate(sample):
        np.testing.assert_allclose(got[b], out_ref[i], rtol=2e-2, atol=2e-3)
        np.testing.assert_allclose(got_z[b], z_ref[i], rtol=2e-2, atol=2e-3)
    # 3. end to end on the GPU's own cache and selection: against the oracle
    # re-run on that selection (its own cache), every sampled row
    _, out_e2e = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q,
                               np.ascontiguousarray(e2e_sel[sample]), np.ascontiguousarray(e2e_nsel[sample]))
    for i, b in enumerate(sample):
        np.testing.assert_allclose(e2e_out[b], out_e2e[i], rtol=2e-2, atol=2e-3)
    same = sum(np.array_equal(e2e_sel[b], o_sel[i]) for i, b in enumerate(sample))
    print(f"[fullsize] {name}: {len(sample)} sampled rows, {same} with the oracle's own selection", flush=True)


def test_llama8b_share_32k_full(gc):
    _decode_full(gc, "llama8b_32k", [0, 2, 5, 7, 9, 11, 13, 15])


def test_llama70b_share_128k_full(gc):
    # the first and last rows and six between (eight of 32)
    _decode_full(gc, "llama70b_128k", [0, 4, 9, 13, 18, 22, 27, 31])


def test_ragged_mix_full(gc):
    w = configs.get("ragged_mix")
    lengths = synth.make_lengths(w)
    # the shortest and the longest sequence, and six more across the batch
    sample = sorted({int(np.argmin(lengths)), int(np.argmax(lengths)), 0, 9, 21, 34, 47, 63})
    _decode_full(gc, "ragged_mix", sample)


def test_prefill_8k_full(gc):
    import routed_decode_attention_amd as rda
    w = configs.get("prefill_8k")
    n, chunk = w.ctx, w.prefill_chunk
    fac = synth.make_factors(w)
    lengths = np.array([n], np.int32)
    pt, total = synth.make_page_table(w, lengths)
    K, V = synth.make_sequence(w, fac, 0, n)
    qp = synth.make_queries(w, n_rows=n)
    d = gc.dims_of(w, 1, total)
    f = rda.Factors(B=gc.dev(fac.B, 0), P=gc.dev(fac.P, 0), R_enc=gc.dev(fac.R_enc, 0),
                    R_dec=gc.dev(fac.R_dec, 0))
    f.W_ofT = torch.empty((w.d_model, w.n_q_heads * w.rank_v), dtype=d.torch_dtype, device="cuda")
    rda.basiskv_fold_output(d, f.B, gc.dev(fac.W_O, w.dtype), f.W_ofT)
    cache = rda.Cache.empty(d, torch.from_numpy(pt))
    ws = rda.new_workspace(d, chunk)
    zs, outs = [], []
    for a in range(0, n, chunk):
        z = torch.empty((chunk, w.n_q_heads, w.rank_v), device="cuda")
        out = torch.empty((chunk, w.d_model), device="cuda")
        rda.basiskv_prefill(d, f, cache, 0, a, gc.dev(qp[a:a + chunk], w.dtype), gc.dev(K[a:a + chunk], w.dtype),
                            gc.dev(V[a:a + chunk], w.dtype), ws, out, z_out=z)
        zs.append(gc.host(z))
        outs.append(gc.host(out))
    torch.cuda.synchronize()
    z_all, out_all = np.concatenate(zs).astype(np.float64), np.concatenate(outs).astype(np.float64)

    od = oracle.Dims.of(w, batch=1, num_pages=total)
    ora = oracle.Cache(od, pt)
    oracle.write(od, fac, ora, 0, 0, K, V)
    W = oracle.fold(od, fac.B, fac.W_O)
    rows = sorted(set(synth.sample_rows(n, 40, seed=3)) | {0, chunk - 1, chunk, n - 1})
    z_ref, out_ref = oracle.attend_causal(od, W, ora, 0, rows, qp[rows])
    np.testing.assert_allclose(z_all[rows], z_ref, rtol=2e-2, atol=2e-3)
    np.testing.assert_allclose(out_all[rows], out_ref, rtol=2e-2, atol=2e-3)
