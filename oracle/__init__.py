"""ctypes front end of the plain fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never imports, links or calls it; the two share no code.  Inputs come from
the seeded generator in ``workloads``; outputs are numpy arrays (fp64 for
results, storage dtype for the cache).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from workloads.configs import BF16, F32, Workload

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.environ.get("BASISKV_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")


def compile_to(src: str, lib: str, werror: bool = True) -> str:
    """gcc build of an oracle source (IEEE fp64, no contraction, OpenMP)."""
    tmp = lib + ".tmp"
    subprocess.check_call([
        "gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"] + (["-Werror"] if werror else [])
        + ["-Wno-unused-parameter", "-I", _HERE, "-o", tmp, src, "-lm"], cwd=_HERE)
    os.replace(tmp, lib)
    return lib


def build(force: bool = True) -> str:
    """Compile liboracle.so (skipped when it exists and ``force`` is false)."""
    if force or not os.path.exists(_LIB):
        compile_to(_SRC, _LIB)
    return _LIB


class _Dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "rank_v", "rank_k",
        "page_size", "d_model", "top_k", "max_pages", "num_pages", "dtype")] + [
        ("scale", C.c_double), ("sink_pages", C.c_int32), ("local_pages", C.c_int32),
        ("group_mean", C.c_int32), ("head_select", C.c_int32)]


class _Cache(C.Structure):
    _fields_ = [("K", C.c_void_p), ("Z", C.c_void_p), ("S", C.c_void_p),
                ("summ", C.c_void_p), ("page_table", C.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = C.CDLL(_LIB)
        p = C.c_void_p
        i32 = C.c_int32
        D = C.POINTER(_Dims)
        Cc = C.POINTER(_Cache)
        lib.ora_round_bf16.argtypes = [C.c_double]
        lib.ora_round_bf16.restype = C.c_uint16
        lib.ora_fold.argtypes = [D, p, p, p]
        lib.ora_write.argtypes = [D, p, p, p, Cc, i32, i32, i32, p, p]
        lib.ora_route.argtypes = [D, p, p, Cc, p, p, p, p, p]
        lib.ora_decode.argtypes = [D, p, Cc, p, p, p, p, p, p]
        lib.ora_attend_causal.argtypes = [D, p, Cc, i32, p, i32, p, p, p]
        for f in ("ora_fold", "ora_write", "ora_route", "ora_decode", "ora_attend_causal"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


@dataclass
class Dims:
    """Shape of one call; mirrors the fields of ora_dims."""

    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rank_v: int
    rank_k: int
    page_size: int
    d_model: int
    top_k: int
    max_pages: int
    num_pages: int
    dtype: int
    scale: float
    sink_pages: int = 0
    local_pages: int = 0
    group_mean: int = 0
    head_select: int = 0

    @classmethod
    def of(cls, w: Workload, **kw) -> "Dims":
        base = dict(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                    head_dim=w.head_dim, rank_v=w.rank_v, rank_k=w.rank_k,
                    page_size=w.page_size, d_model=w.d_model, top_k=w.top_k,
                    max_pages=w.max_pages_per_seq, num_pages=0, dtype=w.dtype,
                    scale=w.softmax_scale, sink_pages=w.sink_pages, local_pages=w.local_pages,
                    group_mean=w.group_mean, head_select=w.head_select)
        base.update(kw)
        return cls(**base)

    def c(self) -> _Dims:
        return _Dims(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                     self.rank_v, self.rank_k, self.page_size, self.d_model,
                     self.top_k, self.max_pages, self.num_pages, self.dtype, self.scale,
                     self.sink_pages, self.local_pages, self.group_mean, self.head_select)

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == F32 else np.uint16

    @property
    def units(self) -> int:
        """Selection units per sequence: KV heads, or query heads with head_select."""
        return self.n_q_heads if self.head_select else self.n_kv_heads


class Cache:
    """Host-resident paged cache in the library's layout."""

    def __init__(self, d: Dims, page_table: np.ndarray, fill=0):
        H, ps = d.n_kv_heads, d.page_size
        dt = d.np_dtype
        self.d = d
        self.K = np.full((d.num_pages, H, ps, d.head_dim), fill, dt)
        self.Z = np.full((d.num_pages, H, d.rank_v, ps), fill, dt)
        self.S = np.full((d.num_pages, H, ps, d.rank_k), fill, dt)
        self.summ = np.zeros((d.num_pages, H, d.rank_v + d.rank_k), np.float32)
        self.page_table = np.ascontiguousarray(page_table, dtype=np.int32)
        assert self.page_table.shape == (d.batch, d.max_pages)

    def c(self) -> _Cache:
        return _Cache(_ptr(self.K), _ptr(self.Z), _ptr(self.S), _ptr(self.summ),
                      _ptr(self.page_table))

    def copy(self) -> "Cache":
        new = Cache.__new__(Cache)
        new.d = self.d
        for n in ("K", "Z", "S", "summ", "page_table"):
            setattr(new, n, getattr(self, n).copy())
        return new


def set_threads(n: int) -> None:
    """OpenMP threads the oracle's loops use from now on (calling thread)."""
    _load()
    C.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def round_bf16(x: float) -> int:
    return int(_load().ora_round_bf16(float(x)))


def fold(d: Dims, B: np.ndarray, W_O: np.ndarray) -> np.ndarray:
    """W_of^T [d_model][H_q*r] in storage dtype."""
    out = np.zeros((d.d_model, d.n_q_heads * d.rank_v), d.np_dtype)
    B = np.ascontiguousarray(B, np.float32)
    W_O = np.ascontiguousarray(W_O, d.np_dtype)
    _load().ora_fold(C.byref(d.c()), _ptr(B), _ptr(W_O), _ptr(out))
    return out


def write(d: Dims, fac, cache: Cache, seq: int, start: int, k: np.ndarray, v: np.ndarray):
    """Write tokens [start, start+len(k)) of row `seq`; k, v [n][H_kv][d_h]."""
    k = np.ascontiguousarray(k, d.np_dtype)
    v = np.ascontiguousarray(v, d.np_dtype)
    n = k.shape[0]
    B = np.ascontiguousarray(fac.B, np.float32)
    P = np.ascontiguousarray(fac.P, np.float32)
    Re = np.ascontiguousarray(fac.R_enc, np.float32)
    cc = cache.c()
    _load().ora_write(C.byref(d.c()), _ptr(B), _ptr(P), _ptr(Re), C.byref(cc),
                      seq, start, n, _ptr(k), _ptr(v))


def route(d: Dims, fac, cache: Cache, seq_lens: np.ndarray, q: np.ndarray):
    """Returns sel [B][U][top_k], n_sel [B][U], scores [B][U][max_pages] with
    U = d.units selection units per sequence."""
    U = d.units
    sel = np.full((d.batch, U, d.top_k), -1, np.int32)
    n_sel = np.zeros((d.batch, U), np.int32)
    scores = np.zeros((d.batch, U, d.max_pages), np.float32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    q = np.ascontiguousarray(q, d.np_dtype)
    P = np.ascontiguousarray(fac.P, np.float32)
    Rd = np.ascontiguousarray(fac.R_dec, np.float32)
    cc = cache.c()
    _load().ora_route(C.byref(d.c()), _ptr(P), _ptr(Rd), C.byref(cc), _ptr(sl), _ptr(q),
                      _ptr(sel), _ptr(n_sel), _ptr(scores))
    return sel, n_sel, scores


def decode(d: Dims, W_ofT: np.ndarray, cache: Cache, seq_lens, q, sel, n_sel):
    """Returns z_out [B][H_q][r] and out [B][d_model], both fp64."""
    z = np.zeros((d.batch, d.n_q_heads, d.rank_v))
    out = np.zeros((d.batch, d.d_model))
    args = [np.ascontiguousarray(a, t) for a, t in (
        (W_ofT, d.np_dtype), (seq_lens, np.int32), (q, d.np_dtype), (sel, np.int32),
        (n_sel, np.int32))]
    cc = cache.c()
    _load().ora_decode(C.byref(d.c()), _ptr(args[0]), C.byref(cc), _ptr(args[1]),
                       _ptr(args[2]), _ptr(args[3]), _ptr(args[4]), _ptr(z), _ptr(out))
    return z, out


def attend_causal(d: Dims, W_ofT, cache: Cache, seq: int, positions: Sequence[int], q):
    """Causal attention for the given query positions; q [n][H_q][d_h]."""
    pos = np.ascontiguousarray(positions, np.int32)
    n = len(pos)
    z = np.zeros((n, d.n_q_heads, d.rank_v))
    out = np.zeros((n, d.d_model))
    W = np.ascontiguousarray(W_ofT, d.np_dtype)
    q = np.ascontiguousarray(q, d.np_dtype)
    cc = cache.c()
    _load().ora_attend_causal(C.byref(d.c()), _ptr(W), C.byref(cc), seq, _ptr(pos), n,
                              _ptr(q), _ptr(z), _ptr(out))
    return z, out


def prefill(d: Dims, fac, W_ofT, cache: Cache, seq: int, start: int, q, k, v):
    """Write a chunk then attend causally for each of its queries."""
    write(d, fac, cache, seq, start, k, v)
    return attend_causal(d, W_ofT, cache, seq, np.arange(start, start + k.shape[0]), q)
