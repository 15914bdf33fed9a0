"""The decode path captured in a HIP graph: a graph holding the fused decode
step and the separate route -> decode calls is replayed several times, with
eager calls of the library, other device work and synchronisations between
the replays.  Every replay must reproduce the eager results bit for bit (the
library records no memset node)."""
import numpy as np
import pytest
import torch

from tests import cases, gpu_cases as gc
from workloads import configs

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager_calls():
    import routed_decode_attention_amd as rda
    w = configs.get("llama8b_32k").with_(name="graph", cfg_id=330, batch=5, top_k=6, d_model=256)
    sc = cases.make_scenario(w, lengths=[700, 1, 130, 64, 513], upto_last=True)
    g = gc.upload(sc, W_ofT=sc.W_ofT)
    gc.write_all(g, sc, upto_last=True, chunk=300)
    B, H, K = sc.batch, g.d.n_kv_heads, g.d.top_k
    kn = gc.dev(np.stack([sc.K[b][int(sc.lengths[b]) - 1][None] for b in range(B)]), w.dtype)
    vn = gc.dev(np.stack([sc.V[b][int(sc.lengths[b]) - 1][None] for b in range(B)]), w.dtype)
    pos = torch.from_numpy(np.asarray(sc.lengths, np.int32) - 1).cuda()
    ws2 = rda.new_workspace(g.d)

    def buffers():
        return dict(sel=torch.full((B, H, K), -7, dtype=torch.int32, device="cuda"),
                    n_sel=torch.full((B, H), -7, dtype=torch.int32, device="cuda"),
                    scores=torch.zeros((B, H, g.d.max_pages_per_seq), device="cuda"),
                    out=torch.zeros((B, g.d.d_model), device="cuda"),
                    z=torch.zeros((B, g.d.n_q_heads, g.d.rank_v), device="cuda"),
                    sel2=torch.full((B, H, K), -7, dtype=torch.int32, device="cuda"),
                    n_sel2=torch.full((B, H), -7, dtype=torch.int32, device="cuda"),
                    scores2=torch.zeros((B, H, g.d.max_pages_per_seq), device="cuda"),
                    phys2=torch.full((B, H, K), -7, dtype=torch.int32, device="cuda"),
                    out2=torch.zeros((B, g.d.d_model), device="cuda"))

    def calls(o, stream=None):
        # the fused step (append + route, attention, merge + projection) ...
        rda.basiskv_decode_step(g.d, g.f, g.cache, pos, kn, vn, g.seq_lens, g.q, o["sel"], o["n_sel"],
                                o["scores"], g.ws, o["out"], z_out=o["z"], stream=stream)
        # ... and the separate calls on the cache it leaves, another workspace
        rda.basiskv_route(g.d, g.f, g.cache, g.seq_lens, g.q, o["sel2"], o["n_sel2"], o["scores2"],
                          sel_phys=o["phys2"], stream=stream)
        rda.basiskv_decode(g.d, g.f, g.cache, g.seq_lens, g.q, o["sel2"], o["n_sel2"], ws2, o["out2"],
                           sel_phys=o["phys2"], stream=stream)

    npg = [-(-int(n) // g.d.page_size) for n in sc.lengths]

    def defined(k, a):
        """Scores are defined for a row's pages only; the rest is unspecified."""
        if not k.startswith("scores"):
            return a
        return np.concatenate([a[b, :, :npg[b]].ravel() for b in range(B)])

    eager = buffers()
    calls(eager)
    torch.cuda.synchronize()
    ref = {k: defined(k, gc.host(v)) for k, v in eager.items()}
    assert np.array_equal(ref["sel"], ref["sel2"]) and np.array_equal(ref["out"], ref["out2"])

    cap = buffers()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            calls(cap, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for rep in range(4):
        for v in cap.values():  # poison the outputs between replays
            v.fill_(-3)
        graph.replay()
        torch.cuda.synchronize()
        for k, v in cap.items():
            assert np.array_equal(defined(k, gc.host(v)), ref[k]), (rep, k)
        # eager work between replays: the library on the same cache and
        # workspaces, then unrelated device work
        other = buffers()
        calls(other)
        torch.cuda.synchronize()
        assert np.array_equal(gc.host(other["out"]), ref["out"]), rep
        torch.randn(1 << 20, device="cuda").sum().item()
