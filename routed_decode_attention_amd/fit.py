"""Offline fitting of the per-KV-head factors from calibration Keys and
Values, and the routing-quality measure.  Host-side numpy, run once before
serving; the decode path itself never calls it.

The pages (weekinpapers "BasisKV: Value Latents for Communication and Key
Routing", Abstract; kongchang article, sections on Value-latent Key routing
and on fitting jointly rather than per partition) state what the factors are
for -- a low-rank Value basis, a predictor of the Key from the Value latent,
and a low-rank Key residual that stores what the latent cannot predict --
but give no fitting procedure.  The plainest least-squares reading, per KV
head:

* B: the r leading right singular vectors of the calibration Values (the
  rank-r subspace that keeps the most Value energy), so z = v.B;
* P: the least-squares map from the latents to the Keys, min ||Z.P - K||;
* R_enc, R_dec: the r_k leading right singular vectors of the residual
  E = K - Z.P and their transpose, the best rank-r_k code of what is left.

The joint objective across tensor-parallel partitions (fitting every GPU's
factors together against the full attention output) is not built here.

Routing quality: for a query head, page j of a sequence holds the exact
softmax mass m_j = sum over its tokens of softmax(scale * q.k)_t; a
selection's recall is the mass its pages hold (1 when every page is kept).
"""
from typing import Dict, Optional

import numpy as np


def _leading_right_vectors(X: np.ndarray, k: int) -> np.ndarray:
    """[d][k]: the k leading right singular vectors of X [n][d] (columns)."""
    _, _, vt = np.linalg.svd(X, full_matrices=False)
    return vt[:k].T


def fit_factors(K: np.ndarray, V: np.ndarray, rank_v: int, rank_k: int) -> Dict[str, np.ndarray]:
    """Factors per KV head from calibration tokens K, V [n][H_kv][d_h]
    (any float dtype).  Returns fp32 B [H][d_h][r], P [H][r][d_h],
    R_enc [H][d_h][r_k], R_dec [H][r_k][d_h] in the library's layout."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n, H, D = V.shape
    if K.shape != V.shape:
        raise ValueError("K and V must have the same shape [n][H_kv][d_h]")
    if not (1 <= rank_v <= D and 1 <= rank_k <= D and n >= max(rank_v, rank_k)):
        raise ValueError("ranks must lie in [1, d_h] and not exceed the token count")
    out = {"B": np.empty((H, D, rank_v), np.float32), "P": np.empty((H, rank_v, D), np.float32),
           "R_enc": np.empty((H, D, rank_k), np.float32), "R_dec": np.empty((H, rank_k, D), np.float32)}
    for g in range(H):
        v, k = V[:, g], K[:, g]
        B = _leading_right_vectors(v, rank_v)
        Z = v @ B
        P, *_ = np.linalg.lstsq(Z, k, rcond=None)
        E = k - Z @ P
        Re = _leading_right_vectors(E, rank_k)
        out["B"][g], out["P"][g], out["R_enc"][g], out["R_dec"][g] = B, P, Re, Re.T
    return out


def page_mass(K: np.ndarray, q: np.ndarray, length: int, page_size: int, group: int,
              scale: Optional[float] = None) -> np.ndarray:
    """Exact softmax mass per page for one sequence: K [n][H_kv][d_h] (its
    first `length` tokens are attended), q [H_q][d_h].  Returns
    [H_q][ceil(length / page_size)] with rows summing to 1."""
    K = np.asarray(K, np.float64)[:length]
    q = np.asarray(q, np.float64)
    Hq, D = q.shape
    s = scale if scale is not None else 1.0 / np.sqrt(D)
    npg = -(-length // page_size)
    mass = np.zeros((Hq, npg))
    for h in range(Hq):
        logits = s * (K[:, h // group] @ q[h])
        p = np.exp(logits - logits.max())
        p /= p.sum()
        padded = np.zeros(npg * page_size)
        padded[:length] = p
        mass[h] = padded.reshape(npg, page_size).sum(axis=1)
    return mass


def recall(mass: np.ndarray, pages) -> float:
    """Mean over query heads of the softmax mass the listed pages hold
    (mass: [H_q of one KV head][n_pages]; pages: selected page ids, -1 ignored)."""
    sel = [int(j) for j in pages if j >= 0]
    return float(np.mean(mass[:, sel].sum(axis=1))) if sel else 0.0


def best_recall(mass: np.ndarray, k: int) -> float:
    """The recall of the k pages with the most mass for each head (an upper
    bound for one shared selection per KV head)."""
    top = np.sort(mass, axis=1)[:, ::-1][:, :k]
    return float(np.mean(top.sum(axis=1)))
