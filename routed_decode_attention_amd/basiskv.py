"""ctypes binding of libbasiskv.so (include/basiskv.h), same names as the C ABI.

Argument marshalling only: each wrapper checks that the torch tensors it is
given are CUDA, contiguous, of the right dtype and large enough for the dims,
then passes their device pointers and torch's current stream to the library.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  If the library is not built, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbasiskv.so")

F32 = 0
BF16 = 1

OK, E_NULL, E_DIMS, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_DATA = 0, -1, -2, -3, -4, -5, -6

EXPORTS = (
    "basiskv_version", "basiskv_strerror", "basiskv_last_error", "basiskv_fold_output",
    "basiskv_write", "basiskv_append", "basiskv_route", "basiskv_append_route",
    "basiskv_workspace_bytes", "basiskv_workspace_init", "basiskv_attend", "basiskv_attend_splits",
    "basiskv_project",
    "basiskv_decode", "basiskv_decode_step", "basiskv_decode_step_noalloc", "basiskv_prefill",
    "basiskv_stream_read",
)


class basiskv_dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "rank_v", "rank_k", "page_size",
        "d_model", "top_k", "max_pages_per_seq", "num_phys_pages", "dtype")] + [
        ("softmax_scale", C.c_float), ("sink_pages", C.c_int32), ("local_pages", C.c_int32),
        ("group_mean", C.c_int32), ("head_select", C.c_int32)]


class basiskv_factors(C.Structure):
    _fields_ = [("B", C.c_void_p), ("P", C.c_void_p), ("R_enc", C.c_void_p),
                ("R_dec", C.c_void_p), ("W_ofT", C.c_void_p)]


class basiskv_cache(C.Structure):
    _fields_ = [("K", C.c_void_p), ("Z", C.c_void_p), ("S", C.c_void_p),
                ("summ", C.c_void_p), ("page_table", C.c_void_p)]


class BasisKVError(RuntimeError):
    def __init__(self, code: int, text: str, detail: str):
        super().__init__(f"basiskv error {code} ({text}): {detail}")
        self.code = code


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    lib = C.CDLL(LIB_PATH)
    p, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    D, Fp, Cp = C.POINTER(basiskv_dims), C.POINTER(basiskv_factors), C.POINTER(basiskv_cache)
    sig = {
        "basiskv_version": ([], C.c_int),
        "basiskv_strerror": ([C.c_int], C.c_char_p),
        "basiskv_last_error": ([], C.c_char_p),
        "basiskv_fold_output": ([D, p, p, p, p], C.c_int),
        "basiskv_write": ([D, Fp, Cp, i32, i32, i32, p, p, p], C.c_int),
        "basiskv_append": ([D, Fp, Cp, p, p, p, p], C.c_int),
        "basiskv_route": ([D, Fp, Cp, p, p, p, p, p, p, p], C.c_int),
        "basiskv_append_route": ([D, Fp, Cp, p, p, p, p, p, p, p, p, p, p], C.c_int),
        "basiskv_decode_step": ([D, Fp, Cp, p, p, p, p, p, p, p, p, p, sz, p, p, p], C.c_int),
        "basiskv_decode_step_noalloc": ([D, Fp, Cp, p, p, p, p, p, p, p, p, p, p, p], C.c_int),
        "basiskv_workspace_bytes": ([D, i32], sz),
        "basiskv_workspace_init": ([D, p, sz, p], C.c_int),
        "basiskv_attend_splits": ([D], C.c_int),
        "basiskv_attend": ([D, Cp, p, p, p, p, p, p, sz, p, p], C.c_int),
        "basiskv_project": ([D, Fp, p, i32, p, p], C.c_int),
        "basiskv_decode": ([D, Fp, Cp, p, p, p, p, p, p, sz, p, p, p], C.c_int),
        "basiskv_prefill": ([D, Fp, Cp, i32, i32, i32, p, p, p, p, sz, p, p, p], C.c_int),
        "basiskv_stream_read": ([p, sz, p, i32, p], C.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def _check(rc: int) -> None:
    if rc != OK:
        raise BasisKVError(rc, _lib.basiskv_strerror(rc).decode(),
                           _lib.basiskv_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel: int = 0):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, need {numel}")
    return t.data_ptr()


@dataclass
class Dims:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rank_v: int
    rank_k: int
    page_size: int
    d_model: int
    top_k: int
    max_pages_per_seq: int
    num_phys_pages: int
    dtype: int
    softmax_scale: float = 0.0
    sink_pages: int = 0
    local_pages: int = 0
    group_mean: int = 0
    head_select: int = 0

    def c(self) -> basiskv_dims:
        return basiskv_dims(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                            self.rank_v, self.rank_k, self.page_size, self.d_model, self.top_k,
                            self.max_pages_per_seq, self.num_phys_pages, self.dtype,
                            self.softmax_scale, self.sink_pages, self.local_pages, self.group_mean,
                            self.head_select)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == F32 else torch.bfloat16

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def units(self) -> int:
        """Selection units per sequence: KV heads, or query heads with head_select."""
        return self.n_q_heads if self.head_select else self.n_kv_heads


@dataclass
class Factors:
    """Device factors: B, P, R_enc, R_dec fp32; W_ofT [d_model][H_q*r] storage dtype."""
    B: torch.Tensor
    P: torch.Tensor
    R_enc: torch.Tensor
    R_dec: torch.Tensor
    W_ofT: Optional[torch.Tensor] = None

    def c(self, d: Dims) -> basiskv_factors:
        H, D, R, RK = d.n_kv_heads, d.head_dim, d.rank_v, d.rank_k
        return basiskv_factors(
            _ptr(self.B, "B", torch.float32, H * D * R), _ptr(self.P, "P", torch.float32, H * R * D),
            _ptr(self.R_enc, "R_enc", torch.float32, H * D * RK),
            _ptr(self.R_dec, "R_dec", torch.float32, H * RK * D),
            _ptr(self.W_ofT, "W_ofT", d.torch_dtype, d.d_model * d.n_q_heads * R))


@dataclass
class Cache:
    """Device paged cache in the library's layout."""
    K: torch.Tensor
    Z: torch.Tensor
    S: torch.Tensor
    summ: torch.Tensor
    page_table: torch.Tensor

    @classmethod
    def empty(cls, d: Dims, page_table: torch.Tensor, device="cuda") -> "Cache":
        P, H, ps, dt = d.num_phys_pages, d.n_kv_heads, d.page_size, d.torch_dtype
        return cls(K=torch.zeros((P, H, ps, d.head_dim), dtype=dt, device=device),
                   Z=torch.zeros((P, H, d.rank_v, ps), dtype=dt, device=device),
                   S=torch.zeros((P, H, ps, d.rank_k), dtype=dt, device=device),
                   summ=torch.zeros((P, H, d.rank_v + d.rank_k), dtype=torch.float32, device=device),
                   page_table=page_table.to(device=device, dtype=torch.int32).contiguous())

    def c(self, d: Dims) -> basiskv_cache:
        P, H, ps = d.num_phys_pages, d.n_kv_heads, d.page_size
        dt = d.torch_dtype
        return basiskv_cache(
            _ptr(self.K, "K", dt, P * H * ps * d.head_dim), _ptr(self.Z, "Z", dt, P * H * d.rank_v * ps),
            _ptr(self.S, "S", dt, P * H * ps * d.rank_k),
            _ptr(self.summ, "summ", torch.float32, P * H * (d.rank_v + d.rank_k)),
            _ptr(self.page_table, "page_table", torch.int32, d.batch * d.max_pages_per_seq))


def basiskv_version() -> int:
    return int(_lib.basiskv_version())


def basiskv_fold_output(d: Dims, B: torch.Tensor, W_O: torch.Tensor, W_ofT: torch.Tensor,
                        stream=None) -> None:
    _check(_lib.basiskv_fold_output(
        C.byref(d.c()), _ptr(B, "B", torch.float32, d.n_kv_heads * d.head_dim * d.rank_v),
        _ptr(W_O, "W_O", d.torch_dtype, d.n_q_heads * d.head_dim * d.d_model),
        _ptr(W_ofT, "W_ofT", d.torch_dtype, d.d_model * d.n_q_heads * d.rank_v), _stream(stream)))


def basiskv_write(d: Dims, f: Factors, cache: Cache, seq: int, start: int, k: torch.Tensor,
                  v: torch.Tensor, stream=None) -> None:
    n = k.shape[0]
    need = n * d.n_kv_heads * d.head_dim
    fc, cc = f.c(d), cache.c(d)
    _check(_lib.basiskv_write(C.byref(d.c()), C.byref(fc), C.byref(cc), seq, start, n,
                              _ptr(k, "k", d.torch_dtype, need), _ptr(v, "v", d.torch_dtype, need),
                              _stream(stream)))


def basiskv_append(d: Dims, f: Factors, cache: Cache, pos: torch.Tensor, k_new: torch.Tensor,
                   v_new: torch.Tensor, stream=None) -> None:
    need = d.batch * d.n_kv_heads * d.head_dim
    fc, cc = f.c(d), cache.c(d)
    _check(_lib.basiskv_append(C.byref(d.c()), C.byref(fc), C.byref(cc),
                               _ptr(pos, "pos", torch.int32, d.batch),
                               _ptr(k_new, "k_new", d.torch_dtype, need),
                               _ptr(v_new, "v_new", d.torch_dtype, need), _stream(stream)))


def workspace_bytes(d: Dims, max_prefill_tokens: int = 0) -> int:
    n = int(_lib.basiskv_workspace_bytes(C.byref(d.c()), max_prefill_tokens))
    if n == 0:
        _check(E_DIMS)
    return n


basiskv_workspace_bytes = workspace_bytes


def new_workspace(d: Dims, max_prefill_tokens: int = 0, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of basiskv_workspace_bytes bytes (its router
    counters must start at zero)."""
    return torch.zeros(workspace_bytes(d, max_prefill_tokens), dtype=torch.uint8, device=device)


def basiskv_workspace_init(d: Dims, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.basiskv_workspace_init(C.byref(d.c()), _ptr(ws, "ws", torch.uint8), ws.numel(),
                                       _stream(stream)))


def basiskv_route(d: Dims, f: Factors, cache: Cache, seq_lens: torch.Tensor, q: torch.Tensor,
                  sel: torch.Tensor, n_sel: torch.Tensor, scores: torch.Tensor, sel_phys=None,
                  stream=None) -> None:
    pairs = d.batch * d.units
    fc, cc = f.c(d), cache.c(d)
    _check(_lib.basiskv_route(
        C.byref(d.c()), C.byref(fc), C.byref(cc),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch),
        _ptr(q, "q", d.torch_dtype, d.batch * d.n_q_heads * d.head_dim),
        _ptr(sel, "sel", torch.int32, pairs * d.top_k), _ptr(n_sel, "n_sel", torch.int32, pairs),
        _ptr(scores, "scores", torch.float32, pairs * d.max_pages_per_seq),
        _ptr(sel_phys, "sel_phys", torch.int32, pairs * d.top_k), _stream(stream)))


def basiskv_append_route(d: Dims, f: Factors, cache: Cache, pos: torch.Tensor, k_new: torch.Tensor,
                         v_new: torch.Tensor, seq_lens: torch.Tensor, q: torch.Tensor,
                         sel: torch.Tensor, n_sel: torch.Tensor, scores: torch.Tensor,
                         sel_phys=None, stream=None) -> None:
    pairs = d.batch * d.units
    need = d.batch * d.n_kv_heads * d.head_dim
    fc, cc = f.c(d), cache.c(d)
    _check(_lib.basiskv_append_route(
        C.byref(d.c()), C.byref(fc), C.byref(cc), _ptr(pos, "pos", torch.int32, d.batch),
        _ptr(k_new, "k_new", d.torch_dtype, need), _ptr(v_new, "v_new", d.torch_dtype, need),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch),
        _ptr(q, "q", d.torch_dtype, d.batch * d.n_q_heads * d.head_dim),
        _ptr(sel, "sel", torch.int32, pairs * d.top_k), _ptr(n_sel, "n_sel", torch.int32, pairs),
        _ptr(scores, "scores", torch.float32, pairs * d.max_pages_per_seq),
        _ptr(sel_phys, "sel_phys", torch.int32, pairs * d.top_k), _stream(stream)))


def basiskv_decode_step(d: Dims, f: Factors, cache: Cache, pos, k_new, v_new, seq_lens, q, sel, n_sel,
                        scores, ws, out, z_out=None, stream=None) -> None:
    pairs = d.batch * d.units
    need = d.batch * d.n_kv_heads * d.head_dim
    fc, cc = f.c(d), cache.c(d)
    _check(_lib.basiskv_decode_step(
        C.byref(d.c()), C.byref(fc), C.byref(cc), _ptr(pos, "pos", torch.int32, d.batch),
        _ptr(k_new, "k_new", d.torch_dtype, need), _ptr(v_new, "v_new", d.torch_dtype, need),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch),
        _ptr(q, "q", d.torch_dtype, d.batch * d.n_q_heads * d.head_dim),
        _ptr(sel, "sel", torch.int32, pairs * d.top_k), _ptr(n_sel, "n_sel", torch.int32, pairs),
        _ptr(scores, "scores", torch.float32, pairs * d.max_pages_per_seq),
        _ptr(ws, "ws", torch.uint8), ws.numel(),
        _ptr(z_out, "z_out", torch.float32, d.batch * d.n_q_heads * d.rank_v),
        _ptr(out, "out", torch.float32, d.batch * d.d_model), _stream(stream)))


def basiskv_decode_step_noalloc(d: Dims, f: Factors, cache: Cache, pos, k_new, v_new, seq_lens, q, sel, n_sel,
                                scores, out, z_out=None, stream=None) -> None:
    """basiskv_decode_step on the library's own per-device scratch (no workspace)."""
    pairs = d.batch * d.units
    need = d.batch * d.n_kv_heads * d.head_dim
    fc, cc = f.c(d), cache.c(d)
    _check(_lib.basiskv_decode_step_noalloc(
        C.byref(d.c()), C.byref(fc), C.byref(cc), _ptr(pos, "pos", torch.int32, d.batch),
        _ptr(k_new, "k_new", d.torch_dtype, need), _ptr(v_new, "v_new", d.torch_dtype, need),
        _ptr(seq_lens, "seq_lens", torch.int32, d.batch),
        _ptr(q, "q", d.torch_dtype, d.batch * d.n_q_heads * d.head_dim),
        _ptr(sel, "sel", torch.int32, pairs * d.top_k), _ptr(n_sel, "n_sel", torch.int32, pairs),
        _ptr(scores, "scores", torch.float32, pairs * d.max_pages_per_seq),
        _ptr(z_out, "z_out", torch.float32, d.batch * d.n_q_heads * d.rank_v),
        _ptr(out, "out", torch.float32, d.batch * d.d_model), _stream(stream)))


def attend_splits(d: Dims) -> int:
    n = _lib.basiskv_attend_splits(C.byref(d.c()))
    _check(min(n, 0))
    return n


def basiskv_attend(d: Dims, cache: Cache, seq_lens, q, sel, n_sel, ws, z_out, sel_phys=None,
                   stream=None) -> None:
    """z_out None: the split partials stay in ws (see the header)."""
    pairs = d.batch * d.units
    cc = cache.c(d)
    _check(_lib.basiskv_attend(
        C.byref(d.c()), C.byref(cc), _ptr(seq_lens, "seq_lens", torch.int32, d.batch),
        _ptr(q, "q", d.torch_dtype, d.batch * d.n_q_heads * d.head_dim),
        _ptr(sel, "sel", torch.int32, pairs * d.top_k), _ptr(n_sel, "n_sel", torch.int32, pairs),
        _ptr(sel_phys, "sel_phys", torch.int32, pairs * d.top_k),
        _ptr(ws, "ws", torch.uint8), ws.numel(),
        _ptr(z_out, "z_out", torch.float32, d.batch * d.n_q_heads * d.rank_v), _stream(stream)))


def basiskv_project(d: Dims, f: Factors, z: torch.Tensor, rows: int, out: torch.Tensor,
                    stream=None) -> None:
    kdim = d.n_q_heads * d.rank_v
    fc = f.c(d)
    _check(_lib.basiskv_project(C.byref(d.c()), C.byref(fc), _ptr(z, "z", torch.float32, rows * kdim),
                                rows, _ptr(out, "out", torch.float32, rows * d.d_model),
                                _stream(stream)))


def basiskv_decode(d: Dims, f: Factors, cache: Cache, seq_lens, q, sel, n_sel, ws, out,
                   z_out=None, sel_phys=None, stream=None) -> None:
    pairs = d.batch * d.units
    fc, cc = f.c(d), cache.c(d)
    _check(_lib.basiskv_decode(
        C.byref(d.c()), C.byref(fc), C.byref(cc), _ptr(seq_lens, "seq_lens", torch.int32, d.batch),
        _ptr(q, "q", d.torch_dtype, d.batch * d.n_q_heads * d.head_dim),
        _ptr(sel, "sel", torch.int32, pairs * d.top_k), _ptr(n_sel, "n_sel", torch.int32, pairs),
        _ptr(sel_phys, "sel_phys", torch.int32, pairs * d.top_k),
        _ptr(ws, "ws", torch.uint8), ws.numel(),
        _ptr(z_out, "z_out", torch.float32, d.batch * d.n_q_heads * d.rank_v),
        _ptr(out, "out", torch.float32, d.batch * d.d_model), _stream(stream)))


def basiskv_prefill(d: Dims, f: Factors, cache: Cache, seq: int, start: int, q, k, v, ws, out,
                    z_out=None, stream=None) -> None:
    n = q.shape[0]
    fc, cc = f.c(d), cache.c(d)
    _check(_lib.basiskv_prefill(
        C.byref(d.c()), C.byref(fc), C.byref(cc), seq, start, n,
        _ptr(q, "q", d.torch_dtype, n * d.n_q_heads * d.head_dim),
        _ptr(k, "k", d.torch_dtype, n * d.n_kv_heads * d.head_dim),
        _ptr(v, "v", d.torch_dtype, n * d.n_kv_heads * d.head_dim),
        _ptr(ws, "ws", torch.uint8), ws.numel(),
        _ptr(z_out, "z_out", torch.float32, n * d.n_q_heads * d.rank_v),
        _ptr(out, "out", torch.float32, n * d.d_model), _stream(stream)))


def basiskv_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of the device tensor src once (a bandwidth probe);
    sink (fp32, one per workgroup) receives each workgroup's sum of the
    words read as fp32."""
    if not (src.is_cuda and src.is_contiguous()):
        raise ValueError("src: a contiguous device tensor")
    _check(_lib.basiskv_stream_read(C.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                    _ptr(sink, "sink", torch.float32, sink.numel()), sink.numel(),
                                    _stream(stream)))
