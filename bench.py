"""Routed latent decode benchmark on one MI355X.

One step is one decode layer step of the whole hot path over the batch:
append the new token (cache writer), route (page scores + top-k), gathered
exact-QK attention over the selected pages, and the folded output projection.
The workload is the Llama-3-8B tensor-parallel-8 share at 32K context:
16 sequences, 4 query heads on 1 KV head, head_dim 128, pages of 64, r=32,
r_k=16, top-k 64 of 512 pages, d_model 4096, bf16 storage, synthetic seeded
data.  The cache of one layer (177.5 MiB) fits in the 256 MB Infinity Cache,
so the timed steps rotate over L distinct layer instances (a 32-layer
attention stack) and every step reads its cache from HBM.

Prints one JSON line (rank 0, one GPU).  See --help.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed decode tokens/s per GPU + achieved HBM TB/s (% peak) at 32K ctx"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary (FETCH_SIZE x its measured copy scale + WRITE_SIZE), or None when
    the attention kernel's source has changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "attend_llama8b_32k_counters.md")
    src = os.path.join(ROOT, "routed_decode_attention_amd", "csrc", "attend.hip")
    try:
        text = open(path).read()
        want = re.search(r"attend\.hip sha256: ([0-9a-f]{64})", text).group(1)
        traffic = int(re.search(r"traffic bytes per launch: (\d+)", text).group(1))
    except (OSError, AttributeError):
        return None
    have = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return traffic if have == want else None


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1024, help="timed layer steps (rounded up to whole sweeps)")
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--workload", default="llama8b_32k")
    p.add_argument("--layers", type=int, default=32, help="distinct cache instances rotated over")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="bound on the oracle's timed CPU work")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--kernel-launches", type=int, default=256, help="launches per kernel for per-kernel timing")
    p.add_argument("--top-k", type=int, default=None, help="pages selected per (sequence, KV head) instead of "
                   "the workload's (a top-k sweep; same data)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU sharding is "
                          "described in the design notes but not built", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import routed_decode_attention_amd as rda
    from tests import gpu_cases as gc
    from workloads import accounting, configs, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = configs.get(args.workload)
    if args.top_k is not None:
        w = w.with_(top_k=args.top_k)
    L = args.layers
    B, H, G = w.batch, w.n_kv_heads, w.group
    t0 = time.time()

    # ---- inputs: seeded synthetic data of the workload's shape --------------------
    fac = synth.make_factors(w, args.seed)
    lengths = synth.make_lengths(w, args.seed)
    pt, total = synth.make_page_table(w, lengths, args.seed)
    seqs = [synth.make_sequence(w, fac, b, int(lengths[b]), args.seed) for b in range(B)]
    q_host = synth.make_queries(w, seed=args.seed)
    log(f"generated inputs in {time.time() - t0:.1f}s")

    d = gc.dims_of(w, B, total)
    f = rda.Factors(B=gc.dev(fac.B, 0), P=gc.dev(fac.P, 0), R_enc=gc.dev(fac.R_enc, 0),
                    R_dec=gc.dev(fac.R_dec, 0))
    f.W_ofT = torch.empty((w.d_model, w.n_q_heads * w.rank_v), dtype=d.torch_dtype, device="cuda")
    rda.basiskv_fold_output(d, f.B, gc.dev(fac.W_O, w.dtype), f.W_ofT)
    page_table = torch.from_numpy(pt).cuda()
    base = rda.Cache.empty(d, page_table)
    # the GPU writer fills tokens [0, n-1); the step appends token n-1
    for b in range(B):
        n = int(lengths[b]) - 1
        rda.basiskv_write(d, f, base, b, 0, gc.dev(seqs[b][0][:n], w.dtype), gc.dev(seqs[b][1][:n], w.dtype))
    torch.cuda.synchronize()
    caches = [base] + [rda.Cache(K=base.K.clone(), Z=base.Z.clone(), S=base.S.clone(),
                                 summ=base.summ.clone(), page_table=page_table) for _ in range(L - 1)]
    # every layer instance has its own factors too (W_of alone is 1 MiB a layer), as in a model
    facs = [f] + [rda.Factors(B=f.B.clone(), P=f.P.clone(), R_enc=f.R_enc.clone(), R_dec=f.R_dec.clone(),
                              W_ofT=f.W_ofT.clone()) for _ in range(L - 1)]
    seq_lens = torch.from_numpy(lengths.astype(np.int32)).cuda()
    pos = (seq_lens - 1).contiguous()
    k_new = gc.dev(np.stack([seqs[b][0][int(lengths[b]) - 1] for b in range(B)]), w.dtype)
    v_new = gc.dev(np.stack([seqs[b][1][int(lengths[b]) - 1] for b in range(B)]), w.dtype)
    q = gc.dev(q_host, w.dtype)
    ws = rda.new_workspace(d)
    sel = torch.zeros((B, H, w.top_k), dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, H, w.max_pages_per_seq), dtype=torch.float32, device="cuda")
    z = torch.zeros((B, w.n_q_heads, w.rank_v), dtype=torch.float32, device="cuda")
    out = torch.zeros((B, w.d_model), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"built {L} cache instances of {base.K.numel() * 2 / 2**20 + base.Z.numel() * 2 / 2**20:.0f} MiB "
        f"(K+Z) in {time.time() - t0:.1f}s")

    def step(i):
        rda.basiskv_decode_step(d, facs[i % L], caches[i % L], pos, k_new, v_new, seq_lens, q, sel, n_sel,
                                scores, ws, out, z_out=z)

    # the first step's selection and output, kept for the oracle comparison below
    step(0)
    torch.cuda.synchronize()
    g_sel, g_nsel = gc.host(sel), gc.host(n_sel)

    # ---- throughput: graph-captured sweeps of L layer steps -------------------------
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for i in range(L):
                step(i)
    torch.cuda.current_stream().wait_stream(s)
    # replayed sweep == eager sweep
    graph.replay()
    torch.cuda.synchronize()
    g_out = out.clone()
    for i in range(L):
        step(i)
    torch.cuda.synchronize()
    assert torch.equal(g_out, out), "graph replay differs from eager execution"

    sweeps = max(1, math.ceil(args.steps / L))
    steps = sweeps * L
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    # an event after every sweep (events do not synchronise): the whole run
    # gives the rate, the sweeps its spread
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(sweeps + 1)]
    t_wall = time.time()
    evs[0].record()
    for k in range(sweeps):
        graph.replay()
        evs[k + 1].record()
    torch.cuda.synchronize()
    t_wall = time.time() - t_wall
    ms = evs[0].elapsed_time(evs[-1])
    sweep_us = np.array([evs[k].elapsed_time(evs[k + 1]) * 1e3 / L for k in range(sweeps)])
    sweep_stats = {"sweeps": sweeps, "median_us_per_step": round(float(np.median(sweep_us)), 3),
                   "p10_us_per_step": round(float(np.percentile(sweep_us, 10)), 3),
                   "p90_us_per_step": round(float(np.percentile(sweep_us, 90)), 3)}
    ms_per_step = ms / steps
    tokens_per_s = B * steps / (ms / 1e3)
    log(f"{steps} steps in {ms:.2f} ms (wall {t_wall * 1e3:.1f} ms): {ms_per_step * 1e3:.2f} us/step, "
        f"{tokens_per_s / 1e6:.3f} M tokens/s per layer step")

    # ---- per-kernel launch durations, live: n back-to-back launches between two
    # events on the stream they run on, queued while the GPU spins so that no
    # host gap enters (the mean agrees with rocprofv3's kernel durations) ----
    def time_launches(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2.0e8))  # ~0.1 s of GPU spin while the launches are queued
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n  # us per launch

    sel_phys = torch.zeros_like(sel)
    rda.basiskv_route(d, f, caches[0], seq_lens, q, sel, n_sel, scores, sel_phys=sel_phys)
    sel_fixed, nsel_fixed, phys_fixed = sel.clone(), n_sel.clone(), sel_phys.clone()
    n_launch = args.kernel_launches
    # the attention kernel as the decode step runs it: physical page ids from
    # the router, split partials left in the workspace (their merge is fused
    # into the projection)
    t_attend = time_launches(lambda i: rda.basiskv_attend(d, caches[i % L], seq_lens, q, sel_fixed,
                                                          nsel_fixed, ws, None, sel_phys=phys_fixed), n_launch)
    t_route = time_launches(lambda i: rda.basiskv_append_route(d, facs[i % L], caches[i % L], pos, k_new, v_new,
                                                               seq_lens, q, sel, n_sel, scores,
                                                               sel_phys=sel_phys, ws=ws), n_launch)
    # attention + the merge fused into the projection, as the step runs them
    t_decode = time_launches(lambda i: rda.basiskv_decode(d, facs[i % L], caches[i % L], seq_lens, q, sel_fixed, nsel_fixed,
                                                          ws, out, sel_phys=phys_fixed), n_launch)
    t_project = t_decode - t_attend

    sb = accounting.decode_step_bytes(w, lengths, selections=gc.host(sel_fixed), n_selected=gc.host(nsel_fixed))
    attend_bytes = sb.attend_kernel
    att_us = float(t_attend)
    achieved = attend_bytes / (att_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "kernel": "attend_mfma_kernel<128,64,32>", "bytes_per_launch": attend_bytes,
                "avg_launch_us": round(att_us, 3), "launches": n_launch}
    # achievable read bandwidth: passes over 4 GiB (16x the Infinity Cache),
    # the best of a few grid sizes
    probe = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
    best = (0.0, 0)
    for n_wg in (256, 512, 1024, 4096, 8192, 16384):
        sink = torch.empty(n_wg, dtype=torch.float32, device="cuda")
        t_read = time_launches(lambda i: rda.basiskv_stream_read(probe, sink), 8)
        best = max(best, (probe.numel() / (t_read * 1e-6) / 1e9, n_wg))
    achievable = best[0]
    del probe
    roofline["achievable_read_GBs"] = round(achievable, 1)
    roofline["frac_of_achievable"] = round(achieved / achievable, 4)
    log(f"achievable HBM read (stream probe, 4 GiB, best grid {best[1]} workgroups): {achievable:.0f} GB/s; "
        f"the attention kernel reaches {100 * achieved / achievable:.1f}% of it")
    step_tbs = sb.total / (ms_per_step * 1e-3) / 1e12
    log(f"attend {att_us:.2f} us ({achieved:.0f} GB/s, {100 * achieved / HBM_PEAK_GBS:.1f}% of 8 TB/s); "
        f"append+route {t_route:.2f} us, merge+project {t_project:.2f} us")

    # ---- CPU baseline: the oracle timed on the same workload; its outputs are
    # also the parity reference of the GPU step ----------------------------------
    cpu, parity = None, None
    if not args.no_cpu:
        import oracle
        from tests import cases
        cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        full = cases.make_scenario(w, seed=args.seed, upto_last=True)
        kn = np.stack([full.K[b][int(lengths[b]) - 1:int(lengths[b])] for b in range(B)])
        vn = np.stack([full.V[b][int(lengths[b]) - 1:int(lengths[b])] for b in range(B)])
        res_o = {}

        def ostep():
            for b in range(B):
                oracle.write(full.d, full.fac, full.cache, b, int(lengths[b]) - 1, kn[b], vn[b])
            s_, n_, sc_ = oracle.route(full.d, full.fac, full.cache, full.lengths, full.q)
            z_, o_ = oracle.decode(full.d, full.W_ofT, full.cache, full.lengths, full.q, s_, n_)
            res_o.update(sel=s_, n_sel=n_, scores=sc_, out=o_)

        reps, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and reps < 100000:
            t1 = time.perf_counter()
            ostep()
            t_cpu += time.perf_counter() - t1
            reps += 1
        cpu = {"value": round(B * reps / t_cpu, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"{reps} full decode layer steps (append+route+decode+project, batch {B}) "
                         f"of the same workload, {t_cpu:.1f} s",
               "ms_per_step": round(t_cpu / reps * 1e3, 2)}
        log(f"oracle: {cpu['value']} tokens/s on {cores} threads ({reps} steps)")

        # parity of the GPU step against the oracle's, every row
        for b in range(B):
            k = int(res_o["n_sel"][b, 0])
            assert int(g_nsel[b, 0]) == k
            npg = -(-int(lengths[b]) // w.page_size)
            cases.check_selection_valid(res_o["scores"][b, 0, :npg], g_sel[b, 0, :k], k, 1e-5)
        rda.basiskv_decode(d, f, caches[0], seq_lens, q, torch.from_numpy(res_o["sel"]).cuda(),
                           torch.from_numpy(res_o["n_sel"]).cuda(), ws, out, z_out=z)
        torch.cuda.synchronize()
        got = gc.host(out).astype(np.float64)
        np.testing.assert_allclose(got, res_o["out"], rtol=2e-2, atol=2e-3)
        same = int(sum(np.array_equal(g_sel[b], res_o["sel"][b]) for b in range(B)))
        parity = {"rows": B, "max_abs_err": float(np.abs(got - res_o["out"]).max()),
                  "selection_identical_rows": same,
                  "tolerance": "selection valid top-k up to 1e-5 relative swaps; out rtol 2e-2 atol 2e-3"}
        log(f"parity ok: max |out - oracle| = {parity['max_abs_err']:.2e}, identical selections {same}/{B}")

    res = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: Llama-3-8B TP=8 share decode, batch {B}, {w.n_q_heads}q:{H}kv "
                               f"heads, head_dim {w.head_dim}, context {w.ctx}, pages of {w.page_size}, "
                               f"r={w.rank_v}, r_k={w.rank_k}, top-k {w.top_k}, d_model {w.d_model}; "
                               f"one step = one attention layer; {L} layer instances rotated",
                   "global_batch": B, "seq_len": int(w.ctx), "parallelism": "single GPU",
                   "layers_rotated": L, "graph_captured": True},
        "hbm_step": {"algorithmic_bytes": sb.total, "TB_per_s": round(step_tbs, 3),
                     "frac_of_8TBs": round(step_tbs / 8.0, 4),
                     "frac_of_achievable": round(step_tbs * 1e3 / achievable, 4)},
        "sweep_spread": sweep_stats,
        "kernels_us": {"append_route": round(float(t_route), 3),
                       "attend": round(att_us, 3), "merge_project": round(float(t_project), 3)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
