"""Routed latent decode benchmark on one MI355X.

One step is one decode layer step of the whole hot path over the batch:
append the new token (cache writer), route (page scores + top-k), gathered
exact-QK attention over the selected pages, and the folded output projection.
The headline workload is the Llama-3-8B tensor-parallel-8 share at 32K
context: 16 sequences, 4 query heads on 1 KV head, head_dim 128, pages of 64,
r=32, r_k=16, top-k 64 of 512 pages, d_model 4096, bf16 storage, synthetic
seeded data.  The cache of one layer (177.5 MiB) fits in the 256 MB Infinity
Cache, so the timed steps rotate over L distinct layer instances (a 32-layer
attention stack) and every step reads its cache from HBM.

After the headline, the other workloads are measured as extra records, each
after its own parity check against the oracle on sampled rows: the
Llama-3-70B share at 128K context, the ragged serving mix, and the 8192-token
causal prefill (TFLOP/s against the bf16 matrix-core peak).

Prints one JSON line (one GPU).  See --help.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed decode tokens/s per GPU + achieved HBM TB/s (% peak) at 32K ctx"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix cores, published

DESC = {
    "llama8b_32k": "Llama-3-8B TP=8 share decode",
    "llama70b_128k": "Llama-3-70B TP=8 share long-context decode",
    "ragged_mix": "ragged paged serving mix decode (lengths U[1024, 65536], scattered pages)",
    "prefill_8k": "causal prefill of one 8192-token prompt in chunks of 2048",
    "llama8b_32k_head_select": "Llama-3-8B TP=8 share decode with one page selection per query head "
                               "(top-k 64 per head) instead of per KV head",
}
LAYERS = {"llama8b_32k": 32, "llama70b_128k": 8, "ragged_mix": 10}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_hash(workload: str = "prefill_8k") -> str:
    """sha256 over the library's kernel and host sources (a counter summary
    is valid only for the sources it was taken with); the decode workloads'
    summaries leave out the prefill kernel's source, which they never run."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "routed_decode_attention_amd", "csrc", "*"))):
        if workload != "prefill_8k" and os.path.basename(p) == "prefill.hip":
            continue
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary profiles/<workload>_counters.md (FETCH_SIZE x
    the copy-calibrated scale + WRITE_SIZE), or None when there is none or the
    sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_counters.md")
    try:
        text = open(path).read()
        want = re.search(r"sources sha256: ([0-9a-f]{64})", text).group(1)
        traffic = sum(int(re.search(r"traffic bytes per launch \[" + re.escape(k) + r"\]: (\d+)", text).group(1))
                      for k in kernel.split("+"))  # a step part of two kernels: both launches
    except (OSError, AttributeError):
        return None
    return traffic if source_hash(workload) == want else None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256, help="timed layer steps (exactly)")
    p.add_argument("--warmup", type=int, default=16, help="untimed warm-up layer steps")
    p.add_argument("--repeats", type=int, default=20, help="further timed replays of the steps, for the spread")
    p.add_argument("--workload", default="llama8b_32k")
    p.add_argument("--layers", type=int, default=None, help="distinct cache instances rotated over")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="bound on the oracle's timed CPU work")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extra", action="store_true", help="skip the extra workloads")
    p.add_argument("--extras", default="llama70b_128k,ragged_mix,llama8b_32k_head_select,prefill_8k",
                   help="comma-separated extra workloads to run after the headline one")
    p.add_argument("--no-headline", action="store_true",
                   help="run only the extra workloads (for profiling one of them); prints no JSON line")
    p.add_argument("--kernel-launches", type=int, default=256, help="launches per kernel for per-kernel timing")
    p.add_argument("--top-k", type=int, default=None, help="pages selected per (sequence, KV head) instead of "
                   "the workload's (a top-k sweep; same data)")
    return p.parse_args()


class Decode:
    """One decode workload on the GPU: L layer instances of its cache and
    factors, written by the GPU writer (tokens [0, n-1)); a step appends
    token n-1 and runs the whole path on one instance."""

    def __init__(self, w, L, seed):
        import torch
        import routed_decode_attention_amd as rda
        from tests import gpu_cases as gc
        from workloads import synth
        self.w, self.L = w, L
        t0 = time.time()
        B, H = w.batch, w.units  # selection units per row
        self.fac = fac = synth.make_factors(w, seed)
        self.lengths = lengths = synth.make_lengths(w, seed)
        pt, total = synth.make_page_table(w, lengths, seed)
        self.d = d = gc.dims_of(w, B, total)
        f = rda.Factors(B=gc.dev(fac.B, 0), P=gc.dev(fac.P, 0), R_enc=gc.dev(fac.R_enc, 0),
                        R_dec=gc.dev(fac.R_dec, 0))
        f.W_ofT = torch.empty((w.d_model, w.n_q_heads * w.rank_v), dtype=d.torch_dtype, device="cuda")
        rda.basiskv_fold_output(d, f.B, gc.dev(fac.W_O, w.dtype), f.W_ofT)
        page_table = torch.from_numpy(pt).cuda()
        base = rda.Cache.empty(d, page_table)
        kn, vn = [], []
        for b in range(B):
            n = int(lengths[b])
            K, V = synth.make_sequence(w, fac, b, n, seed)
            rda.basiskv_write(d, f, base, b, 0, gc.dev(K[:n - 1], w.dtype), gc.dev(V[:n - 1], w.dtype))
            kn.append(K[n - 1])
            vn.append(V[n - 1])
            del K, V
        torch.cuda.synchronize()
        self.caches = [base] + [rda.Cache(K=base.K.clone(), Z=base.Z.clone(), S=base.S.clone(),
                                          summ=base.summ.clone(), page_table=page_table) for _ in range(L - 1)]
        # every layer instance has its own factors too (W_of alone is 1 MiB a layer), as in a model
        self.facs = [f] + [rda.Factors(B=f.B.clone(), P=f.P.clone(), R_enc=f.R_enc.clone(), R_dec=f.R_dec.clone(),
                                       W_ofT=f.W_ofT.clone()) for _ in range(L - 1)]
        self.seq_lens = torch.from_numpy(lengths.astype(np.int32)).cuda()
        self.pos = (self.seq_lens - 1).contiguous()
        self.k_new = gc.dev(np.stack(kn), w.dtype)
        self.v_new = gc.dev(np.stack(vn), w.dtype)
        self.q_host = synth.make_queries(w, seed=seed)
        self.q = gc.dev(self.q_host, w.dtype)
        self.ws = rda.new_workspace(d)
        self.sel = torch.zeros((B, H, w.top_k), dtype=torch.int32, device="cuda")
        self.n_sel = torch.zeros((B, H), dtype=torch.int32, device="cuda")
        self.scores = torch.zeros((B, H, w.max_pages_per_seq), dtype=torch.float32, device="cuda")
        self.z = torch.zeros((B, w.n_q_heads, w.rank_v), dtype=torch.float32, device="cuda")
        self.out = torch.zeros((B, w.d_model), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        mib = (base.K.numel() + base.Z.numel()) * 2 / 2 ** 20
        log(f"{w.name}: {L} cache instances of {mib:.0f} MiB (K+Z), built in {time.time() - t0:.1f}s")

    def step(self, i):
        import routed_decode_attention_amd as rda
        j = i % self.L
        rda.basiskv_decode_step(self.d, self.facs[j], self.caches[j], self.pos, self.k_new, self.v_new,
                                self.seq_lens, self.q, self.sel, self.n_sel, self.scores, self.ws, self.out,
                                z_out=self.z)


def time_steps(step, K, W, repeats, out):
    """W eager warm-up steps, then a graph of exactly K steps (layer i mod L);
    the graph's replay is checked against eager execution, timed once between
    events on its stream (the rate), then `repeats` more times (the spread)."""
    import torch
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for i in range(K):
                step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # replayed steps == eager steps
    graph.replay()
    torch.cuda.synchronize()
    g_out = out.clone()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    assert torch.equal(g_out, out), "graph replay differs from eager execution"
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    rep = []
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        rep.append(a.elapsed_time(b) * 1e3 / K)
    return ms, np.array(rep)


def time_launches(fn, n):
    """us per launch: n back-to-back launches between two events on the
    stream they run on, queued while the GPU spins so that no host gap enters
    (the mean agrees with rocprofv3's kernel durations)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.0e8))
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def mp_kernels(w) -> str:
    """The kernel(s) of the split merge and the projection, by the library's
    rule: fused with 2-row groups up to one MFMA row tile (16 rows), fused with
    16-row tiles beyond while the contraction (query heads x r) is at most
    256, else the merge kernel and the projection kernel."""
    if w.batch <= 16:
        return "merge_project_kernel"
    return "merge_project_rows_kernel" if w.n_q_heads * w.rank_v <= 256 else "merge_kernel+project_mfma_kernel"


def decode_kernels(st, launches):
    """Live per-kernel launch durations of the decode step's three kernels
    (append + scores, attention with its selection prologue, merge +
    projection) and their algorithmic bytes per launch.  The scoring launch
    is timed alone (the scores-only form of append_route); the projection as
    the decode call minus the attention it starts with; the attention with
    its selection as the whole step minus the other two.  Returns {name:
    record}."""
    import torch
    import routed_decode_attention_amd as rda
    from tests import gpu_cases as gc
    from workloads import accounting
    w, L, d = st.w, st.L, st.d
    st.step(0)
    sel, nsel = st.sel.clone(), st.n_sel.clone()
    phys = torch.zeros_like(sel)
    rda.basiskv_route(d, st.facs[0], st.caches[0], st.seq_lens, st.q, torch.empty_like(sel),
                      torch.empty_like(nsel), torch.empty_like(st.scores), sel_phys=phys)
    t_step = time_launches(st.step, launches)
    t_score = time_launches(lambda i: rda.basiskv_append_route(
        d, st.facs[i % L], st.caches[i % L], st.pos, st.k_new, st.v_new, st.seq_lens, st.q, None, None,
        st.scores), launches)
    t_attend = time_launches(lambda i: rda.basiskv_attend(d, st.caches[i % L], st.seq_lens, st.q, sel, nsel,
                                                          st.ws, None, sel_phys=phys), launches)
    t_decode = time_launches(lambda i: rda.basiskv_decode(d, st.facs[i % L], st.caches[i % L], st.seq_lens, st.q,
                                                          sel, nsel, st.ws, st.out, sel_phys=phys), launches)
    t_mp = t_decode - t_attend
    sb = accounting.decode_step_bytes(w, st.lengths, selections=gc.host(sel), n_selected=gc.host(nsel))
    b_score = sb.summaries + sb.page_table + sb.queries + sb.append + sb.factors
    recs = {}
    for name, kern, us, by, how in (
            ("append_score", "score_kernel", t_score, b_score, "events"),
            ("attend_select", "attend_mfma_kernel", t_step - t_score - t_mp, sb.attend_kernel,
             "events (step minus scoring minus merge-projection)"),
            ("merge_project", mp_kernels(w), t_mp, sb.w_of + sb.out,
             "events (decode minus attention)")):
        gbs = by / (us * 1e-6) / 1e9
        recs[name] = {"kernel": kern, "avg_launch_us": round(us, 3), "bytes_per_launch": int(by),
                      "GBs": round(gbs, 1), "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4),
                      "traffic": measured_traffic(kern, w.name), "launches": launches, "timing": how}
    return recs, sb


def roofline_of(recs):
    """The dominant kernel's roofline record (the one with the longest launch)."""
    name = max(recs, key=lambda k: recs[k]["avg_launch_us"])
    r = recs[name]
    return {"bound": "hbm", "achieved": r["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": r["frac_of_8TBs"], "traffic": r["traffic"], "kernel": r["kernel"], "step_part": name,
            "bytes_per_launch": r["bytes_per_launch"], "avg_launch_us": r["avg_launch_us"],
            "launches": r["launches"]}


def achievable_read():
    """Achievable HBM read bandwidth: passes over 4 GiB (16x the Infinity
    Cache), the best of a few grid sizes."""
    import torch
    import routed_decode_attention_amd as rda
    probe = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
    best = (0.0, 0)
    for n_wg in (256, 512, 1024, 4096, 8192, 16384):
        sink = torch.empty(n_wg, dtype=torch.float32, device="cuda")
        t_read = time_launches(lambda i: rda.basiskv_stream_read(probe, sink), 8)
        best = max(best, (probe.numel() / (t_read * 1e-6) / 1e9, n_wg))
    del probe
    torch.cuda.empty_cache()
    return best


def sampled_parity(st, rows):
    """The first decode step's outputs on sampled rows against the oracle (its
    own writer and cache for those rows): selections valid top-k sets, and the
    output against the oracle's decode over the GPU's selection."""
    import torch
    import oracle
    from tests import cases
    from tests import gpu_cases as gc
    w = st.w
    sc = cases.make_scenario(w, rows=rows)
    o_sel, o_nsel, o_scores = oracle.route(sc.d, sc.fac, sc.cache, sc.lengths, sc.q)
    st.step(0)
    torch.cuda.synchronize()
    g_sel, g_nsel, g_out = gc.host(st.sel), gc.host(st.n_sel), gc.host(st.out).astype(np.float64)
    sel = np.ascontiguousarray(g_sel[rows])
    nsel = np.ascontiguousarray(g_nsel[rows])
    assert np.array_equal(nsel, o_nsel)
    for i in range(len(rows)):
        npg = -(-int(sc.lengths[i]) // w.page_size)
        for g in range(w.units):
            k = int(o_nsel[i, g])
            cases.check_selection_valid(o_scores[i, g, :npg], sel[i, g, :k], k, 1e-5)
    _, out_ref = oracle.decode(sc.d, sc.W_ofT, sc.cache, sc.lengths, sc.q, sel, nsel)
    np.testing.assert_allclose(g_out[rows], out_ref, rtol=2e-2, atol=2e-3)
    same = int(sum(np.array_equal(sel[i], o_sel[i]) for i in range(len(rows))))
    return {"rows": [int(r) for r in rows], "max_abs_err": float(np.abs(g_out[rows] - out_ref).max()),
            "selection_identical_rows": same,
            "tolerance": "selection valid top-k up to 1e-5 relative swaps; out vs oracle on the GPU's "
                         "selection, rtol 2e-2 atol 2e-3"}


def run_decode(w, L, K, W, repeats, launches, seed, parity_rows):
    st = Decode(w, L, seed)
    parity = sampled_parity(st, parity_rows) if parity_rows else None
    if parity:
        log(f"{w.name}: parity ok on rows {parity['rows']} (max |out - oracle| {parity['max_abs_err']:.2e})")
    ms, rep = time_steps(st.step, K, W, repeats, st.out)
    recs, sb = decode_kernels(st, launches)
    us = ms * 1e3 / K
    B = w.batch
    rec = {"tokens_per_s": round(B * K / (ms / 1e3), 1), "us_per_step": round(us, 3), "steps": K,
           "layers_rotated": L, "algorithmic_bytes": sb.total,
           "TB_per_s": round(sb.total / (us * 1e-6) / 1e12, 3),
           "frac_of_8TBs": round(sb.total / (us * 1e-6) / 1e12 / 8.0, 4),
           "spread": {"repeats": int(len(rep)), "median_us_per_step": round(float(np.median(rep)), 3),
                      "p10_us_per_step": round(float(np.percentile(rep, 10)), 3),
                      "p90_us_per_step": round(float(np.percentile(rep, 90)), 3)},
           "kernels": recs, "roofline": roofline_of(recs), "parity": parity}
    return st, rec


def run_prefill(seed, repeats=5):
    """The 8192-token prompt in chunks of 2048 (write, causal attention,
    projection per chunk), after a parity check on sampled query rows."""
    import torch
    import oracle
    import routed_decode_attention_amd as rda
    from tests import gpu_cases as gc
    from workloads import accounting, configs, synth
    w = configs.get("prefill_8k")
    n, chunk = w.ctx, w.prefill_chunk
    fac = synth.make_factors(w, seed)
    lengths = np.array([n], np.int32)
    pt, total = synth.make_page_table(w, lengths, seed)
    K, V = synth.make_sequence(w, fac, 0, n, seed)
    qp = synth.make_queries(w, n_rows=n, seed=seed)
    d = gc.dims_of(w, 1, total)
    f = rda.Factors(B=gc.dev(fac.B, 0), P=gc.dev(fac.P, 0), R_enc=gc.dev(fac.R_enc, 0), R_dec=gc.dev(fac.R_dec, 0))
    f.W_ofT = torch.empty((w.d_model, w.n_q_heads * w.rank_v), dtype=d.torch_dtype, device="cuda")
    rda.basiskv_fold_output(d, f.B, gc.dev(fac.W_O, w.dtype), f.W_ofT)
    cache = rda.Cache.empty(d, torch.from_numpy(pt))
    ws = rda.new_workspace(d, chunk)
    qd, kd, vd = gc.dev(qp, w.dtype), gc.dev(K, w.dtype), gc.dev(V, w.dtype)
    z = torch.empty((n, w.n_q_heads, w.rank_v), device="cuda")
    out = torch.empty((n, w.d_model), device="cuda")

    def prompt():
        for a in range(0, n, chunk):
            rda.basiskv_prefill(d, f, cache, 0, a, qd[a:a + chunk], kd[a:a + chunk], vd[a:a + chunk], ws,
                                out[a:a + chunk], z_out=z[a:a + chunk])

    prompt()
    torch.cuda.synchronize()
    # parity on sampled query rows of every chunk
    od = oracle.Dims.of(w, batch=1, num_pages=total)
    ora = oracle.Cache(od, pt)
    oracle.write(od, fac, ora, 0, 0, K, V)
    W_ofT = oracle.fold(od, fac.B, fac.W_O)
    rows = sorted(set(synth.sample_rows(n, 24, seed=5)) | {0, chunk - 1, chunk, n - 1})
    _, out_ref = oracle.attend_causal(od, W_ofT, ora, 0, rows, qp[rows])
    got = gc.host(out).astype(np.float64)[rows]
    np.testing.assert_allclose(got, out_ref, rtol=2e-2, atol=2e-3)
    log(f"prefill_8k: parity ok on {len(rows)} query rows (max |out - oracle| {np.abs(got - out_ref).max():.2e})")
    # timing: whole prompts, then the writer and the projection alone
    t = []
    for _ in range(repeats + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        prompt()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3)
    t = np.array(t[1:])
    t_write = time_launches(lambda i: rda.basiskv_write(d, f, cache, 0, (i % 4) * chunk, kd[(i % 4) * chunk:(i % 4 + 1)
                                                                                          * chunk],
                                                        vd[(i % 4) * chunk:(i % 4 + 1) * chunk]), 8)
    zf = z.view(n, -1)
    t_proj = time_launches(lambda i: rda.basiskv_project(d, f, zf[(i % 4) * chunk:], chunk,
                                                         out[(i % 4) * chunk:]), 8)
    fl = [accounting.prefill_flops(w, a, chunk) for a in range(0, n, chunk)]
    total_fl = sum(x["total"] for x in fl)
    attn_fl = sum(x["attention"] for x in fl)
    proj_fl = sum(x["projection"] for x in fl)
    us = float(np.median(t))
    t_attn = us - 4 * (t_write + t_proj)
    rec = {"tokens_per_s": round(n / (us * 1e-6), 1), "us_per_prompt": round(us, 1),
           "TFLOP_per_s": round(total_fl / (us * 1e-6) / 1e12, 1),
           "frac_of_bf16_mfma_peak": round(total_fl / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
           "flops_per_prompt": int(total_fl),
           "attention": {"us": round(t_attn, 1), "flops": int(attn_fl),
                         "TFLOP_per_s": round(attn_fl / (t_attn * 1e-6) / 1e12, 1),
                         "frac_of_bf16_mfma_peak": round(attn_fl / (t_attn * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                         "timing": "prompt minus 4 x (writer + projection)"},
           "projection": {"us_per_chunk": round(t_proj, 1), "flops_per_chunk": int(proj_fl // 4),
                          "TFLOP_per_s": round(proj_fl / 4 / (t_proj * 1e-6) / 1e12, 1),
                          "frac_of_bf16_mfma_peak": round(proj_fl / 4 / (t_proj * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS,
                                                          4)},
           "writer": {"us_per_chunk": round(t_write, 1)},
           "repeats": repeats,
           "parity": {"query_rows": len(rows), "max_abs_err": float(np.abs(got - out_ref).max()),
                      "tolerance": "rtol 2e-2 atol 2e-3"}}
    return rec


def cpu_baseline(st, seconds, seed):
    """The oracle's whole decode step (append + route + decode + project over
    the batch) timed on the host: all threads for `seconds`, then one thread
    for a third of that.  Its results are also the full-batch parity
    reference of the GPU step."""
    import oracle
    from tests import cases
    w, lengths, B = st.w, st.lengths, st.w.batch
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    full = cases.make_scenario(w, seed=seed, upto_last=True)
    kn = np.stack([full.K[b][int(lengths[b]) - 1:int(lengths[b])] for b in range(B)])
    vn = np.stack([full.V[b][int(lengths[b]) - 1:int(lengths[b])] for b in range(B)])
    res = {}

    def ostep():
        for b in range(B):
            oracle.write(full.d, full.fac, full.cache, b, int(lengths[b]) - 1, kn[b], vn[b])
        s_, n_, sc_ = oracle.route(full.d, full.fac, full.cache, full.lengths, full.q)
        _, o_ = oracle.decode(full.d, full.W_ofT, full.cache, full.lengths, full.q, s_, n_)
        res.update(sel=s_, n_sel=n_, scores=sc_, out=o_)

    def timed(bound):
        reps, t = 0, 0.0
        while t < bound and reps < 100000:
            t1 = time.perf_counter()
            ostep()
            t += time.perf_counter() - t1
            reps += 1
        return reps, t

    oracle.set_threads(cores)
    reps, t_cpu = timed(seconds)
    oracle.set_threads(1)
    reps1, t1 = timed(seconds / 3)
    oracle.set_threads(cores)
    cpu = {"value": round(B * reps / t_cpu, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"{reps} full decode layer steps (append+route+decode+project, batch {B}) of the same "
                     f"workload, {t_cpu:.1f} s on {cores} threads; {reps1} steps, {t1:.1f} s on 1 thread",
           "ms_per_step": round(t_cpu / reps * 1e3, 2), "cpu_model": cpu_model(),
           "value_1thread": round(B * reps1 / t1, 1), "ms_per_step_1thread": round(t1 / reps1 * 1e3, 2)}
    return cpu, full, res


def run_extras(args, names):
    """The extra workloads named (each after its own parity check)."""
    import torch
    from workloads import configs
    extra = {}
    for name, rows in (("llama70b_128k", [0, 31]), ("ragged_mix", None), ("llama8b_32k_head_select", [0, 15])):
        if name not in names:
            continue
        we = configs.get("llama8b_32k").with_(name=name, head_select=1) if name.endswith("head_select") \
            else configs.get(name)
        if rows is None:
            from workloads import synth
            ln = synth.make_lengths(we, args.seed)
            rows = sorted({int(np.argmin(ln)), int(np.argmax(ln)), 17})
        Le = LAYERS.get(name, LAYERS["llama8b_32k"])
        ste, rec = run_decode(we, Le, 4 * Le, 2 * Le, 10, min(args.kernel_launches, 64), args.seed, parity_rows=rows)
        rec["workload"] = f"{name}: {DESC[name]}"
        extra[name] = rec
        log(f"{name}: {rec['us_per_step']:.2f} us/step, {rec['tokens_per_s'] / 1e6:.3f} M tokens/s, "
            f"{100 * rec['frac_of_8TBs']:.1f}% of 8 TB/s; kernels (us): " +
            ", ".join(f"{k} {v['avg_launch_us']:.2f}" for k, v in rec["kernels"].items()))
        del ste
        torch.cuda.empty_cache()
    if "prefill_8k" in names:
        pre = run_prefill(args.seed)
        pre["workload"] = f"prefill_8k: {DESC['prefill_8k']}"
        extra["prefill_8k"] = pre
        log(f"prefill_8k: {pre['us_per_prompt']:.0f} us per prompt, {pre['TFLOP_per_s']} TFLOP/s "
            f"({100 * pre['frac_of_bf16_mfma_peak']:.1f}% of the bf16 matrix-core peak); attention "
            f"{pre['attention']['TFLOP_per_s']} TFLOP/s; per chunk: writer {pre['writer']['us_per_chunk']} us, "
            f"projection {pre['projection']['us_per_chunk']} us ({pre['projection']['TFLOP_per_s']} TFLOP/s)")
    return extra


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the build has one GPU's share of "
                          "the tensor-parallel layer and no collectives; how the path would shard is described "
                          "in the design notes", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import routed_decode_attention_amd as rda
    from tests import cases
    from tests import gpu_cases as gc
    from workloads import configs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = configs.get(args.workload)
    if args.top_k is not None:
        w = w.with_(top_k=args.top_k)
    L = args.layers or LAYERS.get(w.name, 8)
    B = w.batch

    if args.no_headline:
        run_extras(args, set(args.extras.split(",")))
        return
    st, head = run_decode(w, L, args.steps, args.warmup, args.repeats, args.kernel_launches, args.seed,
                          parity_rows=None)
    log(f"{w.name}: {head['steps']} steps, {head['us_per_step']:.2f} us/step, "
        f"{head['tokens_per_s'] / 1e6:.3f} M tokens/s per layer step; kernels (us): " +
        ", ".join(f"{k} {v['avg_launch_us']:.2f}" for k, v in head["kernels"].items()))
    best = achievable_read()
    rf = head["roofline"]
    rf["achievable_read_GBs"] = round(best[0], 1)
    rf["frac_of_achievable"] = round(rf["achieved"] / best[0], 4)
    log(f"achievable HBM read (stream probe, 4 GiB, best grid {best[1]} workgroups): {best[0]:.0f} GB/s; "
        f"dominant kernel {rf['kernel']} ({rf['step_part']}) at {100 * rf['frac']:.1f}% of 8 TB/s")

    # ---- CPU baseline; its outputs are the full-batch parity reference --------
    cpu, parity = None, None
    if not args.no_cpu:
        cpu, full, res_o = cpu_baseline(st, args.cpu_seconds, args.seed)
        log(f"oracle: {cpu['value']} tokens/s on {cpu['cores']} threads, {cpu['value_1thread']} on 1 "
            f"({cpu['cpu_model']})")
        st.step(0)
        torch.cuda.synchronize()
        g_sel, g_nsel = gc.host(st.sel), gc.host(st.n_sel)
        assert np.array_equal(g_nsel, res_o["n_sel"])
        for b in range(B):
            for g in range(w.n_kv_heads):
                k = int(res_o["n_sel"][b, g])
                npg = -(-int(st.lengths[b]) // w.page_size)
                cases.check_selection_valid(res_o["scores"][b, g, :npg], g_sel[b, g, :k], k, 1e-5)
        import oracle
        _, out_gsel = oracle.decode(full.d, full.W_ofT, full.cache, full.lengths, full.q, g_sel, g_nsel)
        got = gc.host(st.out).astype(np.float64)
        np.testing.assert_allclose(got, out_gsel, rtol=2e-2, atol=2e-3)
        same = int(sum(np.array_equal(g_sel[b], res_o["sel"][b]) for b in range(B)))
        parity = {"rows": B, "max_abs_err": float(np.abs(got - out_gsel).max()),
                  "selection_identical_rows": same,
                  "tolerance": "selection valid top-k up to 1e-5 relative swaps; out vs the oracle's decode over "
                               "the GPU's selection, rtol 2e-2 atol 2e-3"}
        log(f"parity ok: max |out - oracle| = {parity['max_abs_err']:.2e}, identical selections {same}/{B}")
    del st
    torch.cuda.empty_cache()

    # ---- extra workloads, each after its own parity check -------------------
    extra = {}
    if not args.no_extra and args.workload == "llama8b_32k" and args.top_k is None:
        extra = run_extras(args, set(args.extras.split(",")))

    res = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": head["steps"], "warmup": args.warmup, "ms_per_step": round(head["us_per_step"] / 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {DESC.get(w.name, w.name)}, batch {B}, {w.n_q_heads}q:{w.n_kv_heads}kv "
                               f"heads, head_dim {w.head_dim}, context {w.max_ctx}, pages of {w.page_size}, "
                               f"r={w.rank_v}, r_k={w.rank_k}, top-k {w.top_k}, d_model {w.d_model}; "
                               f"one step = one attention layer; {L} layer instances rotated",
                   "global_batch": B, "seq_len": int(w.max_ctx), "parallelism": "single GPU",
                   "layers_rotated": L, "graph_captured": True},
        "hbm_step": {"algorithmic_bytes": head["algorithmic_bytes"], "TB_per_s": head["TB_per_s"],
                     "frac_of_8TBs": head["frac_of_8TBs"],
                     "frac_of_achievable": round(head["TB_per_s"] * 1e3 / best[0], 4)},
        "sweep_spread": head["spread"],
        "kernels": head["kernels"],
        "roofline": rf,
        "cpu_baseline": cpu,
        "parity": parity,
        "extra": extra,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
