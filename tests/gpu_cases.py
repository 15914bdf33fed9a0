"""GPU-side scaffolding for parity tests: upload seeded host inputs (and the
oracle's cache, where a test wants identical cache contents) into torch
tensors and call the library through its C-ABI binding."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import routed_decode_attention_amd as rda
from workloads.configs import BF16, F32, Workload


def dev(x: np.ndarray, dtype: int) -> torch.Tensor:
    """Host storage array -> device tensor of the storage dtype (bits preserved)."""
    x = np.ascontiguousarray(x)
    if dtype == BF16 and x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    if x.dtype == np.float64:
        x = x.astype(np.float32)
    return torch.from_numpy(x).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dims_of(w: Workload, batch: int, num_pages: int, **kw) -> rda.Dims:
    base = dict(batch=batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                rank_v=w.rank_v, rank_k=w.rank_k, page_size=w.page_size, d_model=w.d_model,
                top_k=w.top_k, max_pages_per_seq=w.max_pages_per_seq, num_phys_pages=num_pages,
                dtype=w.dtype, softmax_scale=0.0, sink_pages=w.sink_pages, local_pages=w.local_pages,
                group_mean=w.group_mean, head_select=w.head_select)
    base.update(kw)
    return rda.Dims(**base)


@dataclass
class Dev:
    w: Workload
    d: rda.Dims
    f: rda.Factors
    cache: rda.Cache
    seq_lens: torch.Tensor
    q: torch.Tensor
    ws: torch.Tensor


def upload(sc, cache: bool = False, W_ofT: Optional[np.ndarray] = None, max_prefill: int = 0,
           seq_lens=None) -> Dev:
    """Device copy of a scenario.  With ``cache`` the oracle's cache is uploaded
    (identical contents); otherwise the device cache starts empty."""
    w = sc.w
    d = dims_of(w, sc.batch, sc.num_pages)
    f = rda.Factors(B=dev(sc.fac.B, F32), P=dev(sc.fac.P, F32), R_enc=dev(sc.fac.R_enc, F32),
                    R_dec=dev(sc.fac.R_dec, F32))
    if W_ofT is not None:
        f.W_ofT = dev(W_ofT, w.dtype)
    else:
        f.W_ofT = torch.empty((w.d_model, w.n_q_heads * w.rank_v), dtype=d.torch_dtype, device="cuda")
        rda.basiskv_fold_output(d, f.B, dev(sc.fac.W_O, w.dtype), f.W_ofT)
    pt = torch.from_numpy(sc.page_table).cuda()
    if cache:
        c = rda.Cache(K=dev(sc.cache.K, w.dtype), Z=dev(sc.cache.Z, w.dtype), S=dev(sc.cache.S, w.dtype),
                      summ=dev(sc.cache.summ, F32), page_table=pt)
    else:
        c = rda.Cache.empty(d, pt)
    lens = sc.lengths if seq_lens is None else seq_lens
    sl = torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    q = dev(sc.q, w.dtype) if sc.q is not None else None
    ws = rda.new_workspace(d, max_prefill)
    return Dev(w=w, d=d, f=f, cache=c, seq_lens=sl, q=q, ws=ws)


def write_all(g: Dev, sc, upto_last: bool = False, chunk: int = 4096) -> None:
    """GPU writer: every token of every row (or all but the last)."""
    for b, n in enumerate(sc.lengths):
        m = int(n) - 1 if upto_last else int(n)
        for a in range(0, m, chunk):
            e = min(m, a + chunk)
            rda.basiskv_write(g.d, g.f, g.cache, b, a, dev(sc.K[b][a:e], g.w.dtype),
                              dev(sc.V[b][a:e], g.w.dtype))


def append_last(g: Dev, sc) -> None:
    """Decode-step append of each row's last token at position n-1."""
    B = sc.batch
    kn = np.stack([sc.K[b][int(sc.lengths[b]) - 1] for b in range(B)])
    vn = np.stack([sc.V[b][int(sc.lengths[b]) - 1] for b in range(B)])
    pos = torch.from_numpy(np.asarray(sc.lengths, np.int32) - 1).cuda()
    rda.basiskv_append(g.d, g.f, g.cache, pos, dev(kn, g.w.dtype), dev(vn, g.w.dtype))


def route(g: Dev, q: Optional[torch.Tensor] = None):
    U = g.d.units
    sel = torch.full((g.d.batch, U, g.d.top_k), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((g.d.batch, U), -7, dtype=torch.int32, device="cuda")
    scores = torch.zeros((g.d.batch, U, g.d.max_pages_per_seq), dtype=torch.float32, device="cuda")
    rda.basiskv_route(g.d, g.f, g.cache, g.seq_lens, g.q if q is None else q, sel, n_sel, scores)
    torch.cuda.synchronize()
    return host(sel), host(n_sel), host(scores)


def decode(g: Dev, sel: np.ndarray, n_sel: np.ndarray, sel_phys: Optional[np.ndarray] = None):
    z = torch.full((g.d.batch, g.d.n_q_heads, g.d.rank_v), float("nan"), device="cuda")
    out = torch.full((g.d.batch, g.d.d_model), float("nan"), device="cuda")
    phys = None if sel_phys is None else torch.from_numpy(sel_phys).cuda()
    rda.basiskv_decode(g.d, g.f, g.cache, g.seq_lens, g.q, torch.from_numpy(sel).cuda(),
                       torch.from_numpy(n_sel).cuda(), g.ws, out, z_out=z, sel_phys=phys)
    torch.cuda.synchronize()
    return host(z).astype(np.float64), host(out).astype(np.float64)


def cache_host(g: Dev):
    c = g.cache
    return dict(K=host(c.K), Z=host(c.Z), S=host(c.S), summ=host(c.summ))


def tol(w: Workload):
    return (2e-2, 2e-3) if w.dtype == BF16 else (1e-4, 1e-4)
