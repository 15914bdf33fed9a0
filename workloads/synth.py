"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no latent projection, no routing, no attention, no
folding of the value basis into the output projection).  Every array is a
plain numpy array; bf16 data is carried as ``uint16`` bit patterns, rounded
from fp32 with round-to-nearest-even (torch's CPU conversion).

Streams (numpy PCG64 seeded through ``SeedSequence``):

* ``[seed, cfg, 0]``    factors, per KV head in order: the Key/Value mixing
  matrix G (d_h x d_h, N(0,1)); a Gaussian d_h x r matrix whose reduced QR
  Q-factor is the value basis B; P (r x d_h, std 1/sqrt(r)); R_enc
  (d_h x r_k, std 1/sqrt(d_h)); R_dec (r_k x d_h, std 1/sqrt(r_k)).  Then the
  output-projection slice W_O (H_q*d_h x d_model, std 1/sqrt(H_q*d_h)).
* ``[seed, cfg, 1, b]`` sequence b, per KV head: V (n x d_h, N(0,1)), noise
  (n x d_h, N(0,1)); K = V.G/sqrt(d_h) + 0.5*noise.  Keys correlate with
  Values through G, as a real layer's do.
* ``[seed, cfg, 2]``    queries, N(0,1).
* ``[seed, cfg, 3]``    physical page placement (identity, or a random
  permutation of the whole pool for scattered workloads).
* ``[seed, cfg, 4]``    ragged lengths, integers uniform in the inclusive range.

The std of the scaled matrices is 1/sqrt(fan_in) with fan_in the number of
input rows of the stored matrix.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from .configs import BF16, F32, Workload


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def to_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float data to the storage dtype (fp32, or bf16 bits as uint16)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x32
    t = torch.from_numpy(x32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def storage_to_f64(x: np.ndarray, dtype: int) -> np.ndarray:
    """Exact widening of stored values to float64."""
    if dtype == F32:
        return np.asarray(x, dtype=np.float64)
    u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


@dataclass
class Factors:
    mix: np.ndarray      # [H_kv][d_h][d_h] float64 (generator only: Key/Value correlation)
    B: np.ndarray        # [H_kv][d_h][r]   float32, orthonormal columns
    P: np.ndarray        # [H_kv][r][d_h]   float32
    R_enc: np.ndarray    # [H_kv][d_h][r_k] float32
    R_dec: np.ndarray    # [H_kv][r_k][d_h] float32
    W_O: np.ndarray      # [H_q*d_h][d_model] storage dtype


def make_factors(w: Workload, seed: int = 0) -> Factors:
    rng = _rng(seed, w.cfg_id, 0)
    D, R, RK, H = w.head_dim, w.rank_v, w.rank_k, w.n_kv_heads
    mix = np.empty((H, D, D))
    B = np.empty((H, D, R), np.float32)
    P = np.empty((H, R, D), np.float32)
    Re = np.empty((H, D, RK), np.float32)
    Rd = np.empty((H, RK, D), np.float32)
    for g in range(H):
        mix[g] = rng.standard_normal((D, D))
        q, _ = np.linalg.qr(rng.standard_normal((D, R)), mode="reduced")
        B[g] = q
        P[g] = rng.standard_normal((R, D)) / np.sqrt(R)
        Re[g] = rng.standard_normal((D, RK)) / np.sqrt(D)
        Rd[g] = rng.standard_normal((RK, D)) / np.sqrt(RK)
    fan = w.n_q_heads * D
    W_O = to_storage(rng.standard_normal((fan, w.d_model)) / np.sqrt(fan), w.dtype)
    return Factors(mix=mix, B=B, P=P, R_enc=Re, R_dec=Rd, W_O=W_O)


def make_lengths(w: Workload, seed: int = 0) -> np.ndarray:
    if w.length_range is None:
        return np.full(w.batch, w.ctx, dtype=np.int32)
    lo, hi = w.length_range
    return _rng(seed, w.cfg_id, 4).integers(lo, hi, endpoint=True, size=w.batch).astype(np.int32)


def make_sequence(w: Workload, fac: Factors, b: int, n: int, seed: int = 0):
    """Keys and Values of sequence b: two arrays [n][H_kv][d_h] in storage dtype.

    ``n`` must be the sequence's full length (the draw order makes prefixes of
    different lengths differ); callers slice what they need.
    """
    rng = _rng(seed, w.cfg_id, 1, b)
    D = w.head_dim
    K = np.empty((n, w.n_kv_heads, D), np.float32)
    V = np.empty((n, w.n_kv_heads, D), np.float32)
    for g in range(w.n_kv_heads):
        v = rng.standard_normal((n, D))
        noise = rng.standard_normal((n, D))
        V[:, g] = v
        K[:, g] = v @ fac.mix[g] / np.sqrt(D) + 0.5 * noise
    return to_storage(K, w.dtype), to_storage(V, w.dtype)


def make_queries(w: Workload, n_rows: Optional[int] = None, seed: int = 0) -> np.ndarray:
    """Queries [rows][H_q][d_h] in storage dtype; rows defaults to the batch."""
    rows = w.batch if n_rows is None else n_rows
    q = _rng(seed, w.cfg_id, 2).standard_normal((rows, w.n_q_heads, w.head_dim))
    return to_storage(q, w.dtype)


def make_page_table(w: Workload, lengths: np.ndarray, seed: int = 0,
                    permuted: Optional[bool] = None):
    """Page table [B][max_pages] int32 (-1 = unmapped) and the pool size.

    The pool holds exactly the pages the sequences need.  Identity placement
    puts sequence b's pages contiguously in order; permuted placement
    scatters every page of the pool by one random permutation.
    """
    ps = w.page_size
    npg = [-(-int(n) // ps) for n in lengths]
    total = int(sum(npg))
    mp = w.max_pages_per_seq
    pt = np.full((len(lengths), mp), -1, dtype=np.int32)
    perm = permuted if permuted is not None else w.permuted_pages
    phys = (_rng(seed, w.cfg_id, 3).permutation(total) if perm
            else np.arange(total)).astype(np.int32)
    off = 0
    for b, c in enumerate(npg):
        pt[b, :c] = phys[off:off + c]
        off += c
    return pt, total


def permute_pool(pt: np.ndarray, total: int, seed: int) -> np.ndarray:
    """A page table with every physical id renamed by a seeded permutation."""
    perm = _rng(seed, 99).permutation(total).astype(np.int32)
    out = pt.copy()
    m = out >= 0
    out[m] = perm[out[m]]
    return out


def sample_rows(n: int, k: int, seed: int) -> List[int]:
    """k distinct sorted indices in [0, n)."""
    k = min(k, n)
    return sorted(_rng(seed, 77).choice(n, size=k, replace=False).tolist())
