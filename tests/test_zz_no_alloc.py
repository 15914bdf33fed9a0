"""The allocation-free decode step (its scratch is the library's own
per-device array) against basiskv_decode_step with a caller workspace: the
same kernels on the same inputs, so every output is bit-identical.  Two
calls in a row, the second with a smaller batch and shorter sequences (the
array keeps the first call's contents), then dims whose workspace exceeds
the array are refused before anything runs."""
import numpy as np
import pytest
import torch

from tests import cases
from workloads import configs

pytestmark = pytest.mark.gpu


def _step(gc, rda, sc, noalloc):
    w = sc.w
    g = gc.upload(sc, W_ofT=sc.W_ofT)
    gc.write_all(g, sc, upto_last=True, chunk=1000)
    B = sc.batch
    kn = gc.dev(np.stack([sc.K[b][int(sc.lengths[b]) - 1] for b in range(B)]), w.dtype)
    vn = gc.dev(np.stack([sc.V[b][int(sc.lengths[b]) - 1] for b in range(B)]), w.dtype)
    pos = torch.from_numpy(np.asarray(sc.lengths, np.int32) - 1).cuda()
    d = g.d
    sel = torch.full((B, d.n_kv_heads, d.top_k), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((B, d.n_kv_heads), -7, dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, d.n_kv_heads, d.max_pages_per_seq), device="cuda")
    z = torch.zeros((B, d.n_q_heads, d.rank_v), device="cuda")
    out = torch.zeros((B, d.d_model), device="cuda")
    if noalloc:
        rda.basiskv_decode_step_noalloc(d, g.f, g.cache, pos, kn, vn, g.seq_lens, g.q, sel, n_sel, scores, out,
                                        z_out=z)
    else:
        rda.basiskv_decode_step(d, g.f, g.cache, pos, kn, vn, g.seq_lens, g.q, sel, n_sel, scores, g.ws, out,
                                z_out=z)
    torch.cuda.synchronize()
    npg = [-(-int(n) // w.page_size) for n in sc.lengths]
    sc_h = gc.host(scores)
    return dict(sel=gc.host(sel), n_sel=gc.host(n_sel), z=gc.host(z), out=gc.host(out),
                scores=[sc_h[b, :, :npg[b]] for b in range(B)], cache=gc.cache_host(g))


def test_noalloc_decode_step_matches_workspace_entry_point():
    assert torch.cuda.is_available()
    import oracle
    import routed_decode_attention_amd as rda
    from tests import gpu_cases as gc
    oracle.build(force=False)
    w = configs.get("llama8b_32k").with_(name="na", cfg_id=501, batch=6, top_k=24, d_model=512)
    big = cases.make_scenario(w, lengths=[3000, 2500, 64, 1, 4097, 1800])
    small = cases.make_scenario(w.with_(batch=3, top_k=8), lengths=[900, 130, 65])
    for i, sc in enumerate((big, small)):
        print(f"[noalloc] call {i}: batch {sc.batch}, lengths {sc.lengths.tolist()}", flush=True)
        a = _step(gc, rda, sc, noalloc=False)
        b = _step(gc, rda, sc, noalloc=True)
        for k in ("sel", "n_sel", "z", "out"):
            assert np.array_equal(a[k], b[k]), k
        for x, y in zip(a["scores"], b["scores"]):
            assert np.array_equal(x, y)
        for k in a["cache"]:
            assert np.array_equal(a["cache"][k], b["cache"][k]), k
        # and both against the oracle, on the GPU's selection
        cases.check_outputs_on_selection(sc, b["sel"], b["n_sel"], b["z"], b["out"])


def test_noalloc_refuses_dims_beyond_its_scratch():
    """Refused on the host before any device access (fake device pointers)."""
    import ctypes as C
    import routed_decode_attention_amd as rda
    from routed_decode_attention_amd import basiskv as bk
    from tests import gpu_cases as gc
    w = configs.get("llama8b_32k")
    d = gc.dims_of(w, 4096, 4096)  # 4096 sequences: the split partials alone exceed the array
    assert rda.workspace_bytes(d) > 4 << 20
    fake = C.c_void_p(0x1000)
    f = bk.basiskv_factors(fake, fake, fake, fake, fake)
    c = bk.basiskv_cache(fake, fake, fake, fake, fake)
    lib = C.CDLL(rda.LIB_PATH)
    rc = lib.basiskv_decode_step_noalloc(C.byref(d.c()), C.byref(f), C.byref(c), *([fake] * 10), None)
    assert rc == -4
    lib.basiskv_last_error.restype = C.c_char_p
    assert b"scratch" in lib.basiskv_last_error()
