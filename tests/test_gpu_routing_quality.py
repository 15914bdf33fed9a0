"""Routing quality with factors fitted offline (PCA / least squares /
truncated SVD of the residual) against the generator's random factors, on
the synthetic workload whose Keys depend on the Values: the GPU router's
selection, scored by the exact softmax mass its pages hold (recall)."""
import numpy as np
import pytest
import torch

from tests import cases, gpu_cases as gc
from workloads import configs, synth
from routed_decode_attention_amd import fit

pytestmark = pytest.mark.gpu


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_fitted_factors_route_to_more_attention_mass():
    import routed_decode_attention_amd as rda
    w = configs.get("llama8b_32k").with_(name="fitq", cfg_id=311, batch=8, top_k=8, d_model=256)
    n = 2048  # 32 pages per sequence, 8 selected
    sc = cases.make_scenario(w, lengths=[n] * w.batch, write=False)
    # calibration tokens: other sequences of the same generator
    cal = [synth.make_sequence(w, sc.fac, 100 + i, n) for i in range(4)]
    Kc = np.concatenate([_f32(k) for k, _ in cal])
    Vc = np.concatenate([_f32(v) for _, v in cal])
    fitted = fit.fit_factors(Kc, Vc, w.rank_v, w.rank_k)
    G = w.n_q_heads // w.n_kv_heads
    masses = [fit.page_mass(_f32(sc.K[b]), _f32(sc.q[b]), n, w.page_size, G) for b in range(w.batch)]
    res = {}
    for name in ("random", "fitted", "fitted, group mean"):
        g = gc.upload(sc)
        if name == "fitted, group mean":
            g.d.group_mean = 1
        if name != "random":
            g.f = rda.Factors(B=torch.from_numpy(fitted["B"]).cuda(), P=torch.from_numpy(fitted["P"]).cuda(),
                              R_enc=torch.from_numpy(fitted["R_enc"]).cuda(),
                              R_dec=torch.from_numpy(fitted["R_dec"]).cuda(), W_ofT=g.f.W_ofT)
        gc.write_all(g, sc)
        sel, n_sel, _ = gc.route(g)
        rec = []
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                assert n_sel[b, h] == w.top_k
                rec.append(fit.recall(masses[b][h * G:(h + 1) * G], sel[b, h]))
        res[name] = float(np.mean(rec))
    best = float(np.mean([fit.best_recall(masses[b][h * G:(h + 1) * G], w.top_k)
                          for b in range(w.batch) for h in range(w.n_kv_heads)]))
    # the same page-mean routing on the exact Keys: the ceiling of what
    # predicted Keys can reach with this score
    exact = []
    for b in range(w.batch):
        Kb, qb = _f32(sc.K[b]).astype(np.float64), _f32(sc.q[b]).astype(np.float64)
        for h in range(w.n_kv_heads):
            means = Kb[:, h].reshape(-1, w.page_size, w.head_dim).mean(axis=1)
            score = (means @ qb[h * G:(h + 1) * G].T).max(axis=1)
            top = np.argsort(-score, kind="stable")[:w.top_k]
            exact.append(fit.recall(masses[b][h * G:(h + 1) * G], top))
    exact = float(np.mean(exact))
    print(f"\nrecall of {w.top_k} of {n // w.page_size} pages: random factors {res['random']:.4f}, "
          f"fitted {res['fitted']:.4f} (group mean instead of max: {res['fitted, group mean']:.4f}), "
          f"page-mean routing on exact Keys {exact:.4f}, best per head {best:.4f}, "
          f"uniform {w.top_k * w.page_size / n:.4f}")
    assert res["fitted"] > res["random"]
    assert res["fitted"] <= best + 1e-9


def _fitted_scenario(w, lengths, cal_seed):
    """A scenario whose factors are fitted to calibration tokens of the same
    generator (other sequences), and the oracle cache written with them."""
    import oracle
    sc = cases.make_scenario(w, lengths=lengths, write=False)
    n = 2048
    cal = [synth.make_sequence(w, sc.fac, cal_seed + i, n) for i in range(4)]
    Kc = np.concatenate([_f32(k) for k, _ in cal])
    Vc = np.concatenate([_f32(v) for _, v in cal])
    f = fit.fit_factors(Kc, Vc, w.rank_v, w.rank_k)
    sc.fac = synth.Factors(mix=sc.fac.mix, B=f["B"], P=f["P"], R_enc=f["R_enc"], R_dec=f["R_dec"], W_O=sc.fac.W_O)
    sc.cache = oracle.Cache(sc.d, sc.page_table)
    for b, m in enumerate(sc.lengths):
        if m > 0:
            oracle.write(sc.d, sc.fac, sc.cache, b, 0, sc.K[b][:m], sc.V[b][:m])
    sc.W_ofT = oracle.fold(sc.d, sc.fac.B, sc.fac.W_O)
    return sc


def test_recall_against_k():
    """Recall of the GPU router's selection as k grows (4, 8, 16 and 32 of
    32 pages), with the generator's random factors and with fitted ones; the
    same score on the exact Keys and the best k pages per head for
    reference.  Selections at a larger k contain those at a smaller one, so
    every column grows with k, and k = 32 keeps all the mass."""
    import routed_decode_attention_amd as rda
    w = configs.get("llama8b_32k").with_(name="fitk", cfg_id=313, batch=8, top_k=32, d_model=256)
    n = 2048
    sc = cases.make_scenario(w, lengths=[n] * w.batch, write=False)
    fitted = _fitted_scenario(w, [n] * w.batch, 100).fac
    G = w.n_q_heads // w.n_kv_heads
    masses = [fit.page_mass(_f32(sc.K[b]), _f32(sc.q[b]), n, w.page_size, G) for b in range(w.batch)]
    ks = (4, 8, 16, 32)
    table = {}
    for name in ("random", "fitted"):
        g = gc.upload(sc)
        if name == "fitted":
            dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
            g.f = rda.Factors(B=dev(fitted.B), P=dev(fitted.P), R_enc=dev(fitted.R_enc), R_dec=dev(fitted.R_dec),
                              W_ofT=g.f.W_ofT)
        gc.write_all(g, sc)
        for k in ks:
            g.d.top_k = k
            sel, n_sel, _ = gc.route(g)
            assert (n_sel == k).all()
            table[name, k] = float(np.mean([fit.recall(masses[b][h * G:(h + 1) * G], sel[b, h])
                                            for b in range(w.batch) for h in range(w.n_kv_heads)]))
    for k in ks:
        exact = []
        for b in range(w.batch):
            Kb, qb = _f32(sc.K[b]).astype(np.float64), _f32(sc.q[b]).astype(np.float64)
            for h in range(w.n_kv_heads):
                means = Kb[:, h].reshape(-1, w.page_size, w.head_dim).mean(axis=1)
                score = (means @ qb[h * G:(h + 1) * G].T).max(axis=1)
                exact.append(fit.recall(masses[b][h * G:(h + 1) * G], np.sort(np.argsort(-score, kind="stable")[:k])))
        table["exact keys", k] = float(np.mean(exact))
        table["best", k] = float(np.mean([fit.best_recall(masses[b][h * G:(h + 1) * G], k)
                                          for b in range(w.batch) for h in range(w.n_kv_heads)]))
    cols = ("random", "fitted", "exact keys", "best")
    print("\nrecall of k of 32 pages (mean over %d sequence x KV-head pairs)" % (w.batch * w.n_kv_heads))
    print("   k  " + "  ".join(f"{c:>10s}" for c in cols) + "    uniform")
    for k in ks:
        print(f"  {k:2d}  " + "  ".join(f"{table[c, k]:10.4f}" for c in cols) + f"  {k / 32:9.4f}")
    for c in cols:
        r = [table[c, k] for k in ks]
        assert all(a <= b + 1e-12 for a, b in zip(r, r[1:])), (c, r)
        assert abs(r[-1] - 1.0) < 1e-9, (c, r)
    for k in ks[:-1]:
        assert table["fitted", k] > table["random", k]
        assert table["fitted", k] <= table["best", k] + 1e-9


def test_fitted_factors_decode_step_matches_oracle():
    """GPU writer, decode-step append, router and decode with fitted factors
    against the oracle run on the same fitted factors: the written cache
    within the writer bound, valid top-k selections, and every row's output
    against the oracle re-run on the GPU's selection."""
    import oracle
    w = configs.get("llama8b_32k").with_(name="fitp", cfg_id=314, batch=4, top_k=8, d_model=256)
    sc = _fitted_scenario(w, [1500, 700, 2048, 65], 300)
    sel, n_sel, scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    g = gc.upload(sc)
    gc.write_all(g, sc, upto_last=True, chunk=500)
    gc.append_last(g, sc)
    torch.cuda.synchronize()
    cases.compare_written(sc, gc.cache_host(g), sc.cache)
    gs, gn, gscores = gc.route(g)
    assert np.array_equal(gn, n_sel)
    for b, n in enumerate(sc.lengths):
        npg = -(-int(n) // w.page_size)
        for h in range(w.n_kv_heads):
            k = int(n_sel[b, h])
            ranked = scores[b, h, :npg].astype(np.float64).copy()
            ranked[[j for j in range(npg) if j < w.sink_pages or j >= npg - w.local_pages]] = np.inf
            cases.check_selection_valid(ranked, gs[b, h, :k], k, 1e-5)
            np.testing.assert_allclose(gscores[b, h, :npg], scores[b, h, :npg], rtol=1e-5,
                                       atol=1e-5 * max(1.0, float(np.abs(scores[b, h, :npg]).max())))
    z, out = gc.decode(g, gs, gn)
    cases.check_outputs_on_selection(sc, gs, gn, z, out)


def test_output_aware_fit_lowers_the_decode_error():
    """The GPU decode (every page selected, so only the Value compression
    acts) against exact dense attention through W_O, with the Value basis
    folded into W_O against the basis and projection fitted to the output, and
    against that basis with every head's projection refitted jointly to the
    layer output of calibration queries."""
    import routed_decode_attention_amd as rda
    w = configs.get("llama8b_32k").with_(name="fito", cfg_id=312, batch=4, top_k=16, d_model=256)
    n = 1024  # 16 pages, all selected
    sc = cases.make_scenario(w, lengths=[n] * w.batch, write=False)
    cal = [synth.make_sequence(w, sc.fac, 200 + i, n) for i in range(4)]
    Kc = np.concatenate([_f32(k) for k, _ in cal])
    Vc = np.concatenate([_f32(v) for _, v in cal])
    W_O = _f32(sc.fac.W_O).astype(np.float64)
    G, D, dm = w.n_q_heads // w.n_kv_heads, w.head_dim, w.d_model
    exact = np.zeros((w.batch, dm))
    for b in range(w.batch):
        Kb, Vb, qb = (_f32(x).astype(np.float64) for x in (sc.K[b], sc.V[b], sc.q[b]))
        for h in range(w.n_q_heads):
            s = Kb[:, h // G] @ qb[h] / np.sqrt(D)
            p = np.exp(s - s.max())
            exact[b] += (p / p.sum()) @ Vb[:, h // G] @ W_O[h * D:(h + 1) * D]
    # the joint fit's calibration outputs: dense attention of 2048 queries
    # (a seed apart from the test's) over each calibration sequence
    nq = 2048
    qc = _f32(synth.make_queries(w, n_rows=nq, seed=7)).astype(np.float64)
    O = []
    for k, v in cal:
        Kb, Vb = _f32(k).astype(np.float64), _f32(v).astype(np.float64)
        o = np.empty((nq, w.n_q_heads, D))
        for h in range(w.n_q_heads):
            s = qc[:, h] @ Kb[:, h // G].T / np.sqrt(D)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            o[:, h] = (p / p.sum(axis=1, keepdims=True)) @ Vb[:, h // G]
        O.append(o)
    O = np.concatenate(O)
    errs = {}
    for name in ("value basis", "output fit", "joint fit"):
        if name == "value basis":
            fac = fit.fit_factors(Kc, Vc, w.rank_v, w.rank_k)
        else:
            fac = fit.fit_output_aware(Kc, Vc, W_O, w.n_q_heads, w.rank_v, w.rank_k)
            if name == "joint fit":  # the output fit's basis, every head's projection refitted together
                fac["W_ofT"] = fit.fit_joint_projection(O, W_O, fac["B"])
        g = gc.upload(sc)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
        g.f = rda.Factors(B=dev(fac["B"]), P=dev(fac["P"]), R_enc=dev(fac["R_enc"]), R_dec=dev(fac["R_dec"]))
        if name == "value basis":
            g.f.W_ofT = torch.empty((dm, w.n_q_heads * w.rank_v), dtype=torch.bfloat16, device="cuda")
            rda.basiskv_fold_output(g.d, g.f.B, gc.dev(sc.fac.W_O, w.dtype), g.f.W_ofT)
        else:
            g.f.W_ofT = dev(fac["W_ofT"]).to(torch.bfloat16)
        gc.write_all(g, sc)
        sel, n_sel, _ = gc.route(g)
        assert (n_sel == n // w.page_size).all()
        _, out = gc.decode(g, sel, n_sel)
        errs[name] = float(np.linalg.norm(out - exact) / np.linalg.norm(exact))
    print(f"\nrelative decode-output error against dense attention (r={w.rank_v} of d_h={D}): "
          f"value basis {errs['value basis']:.4f}, output fit {errs['output fit']:.4f}, "
          f"joint fit {errs['joint fit']:.4f}")
    assert errs["joint fit"] < errs["output fit"] < errs["value basis"]
