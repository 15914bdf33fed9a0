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

Fitting against the attention output instead of the Values (the pages: fit
the factors jointly against the full attention output, the Value basis tied
to the output projection).  A query head h's output is o_h.W_O[h] with o_h a
convex combination of the Values, so over calibration Values X the group's
outputs are X.W_g, W_g = [W_O[h] for the group's heads] (d_h x group*d_model).
The rank-r map X.B.C closest to X.W_g in least squares (reduced-rank
regression) is B = W_g.U_r, C = U_r^T with U_r the r leading right singular
vectors of X.W_g: the latent basis B and, per head, the folded projection
W_of[h] = C's block for h -- passed to the library as W_ofT instead of
folding B^T.W_O (which assumes an orthonormal B).  Across several GPUs'
partitions, fit_joint_projection refits every head's projection together
against the layer's whole output, given the latent bases.

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


def fit_output_aware(K: np.ndarray, V: np.ndarray, W_O: np.ndarray, n_q_heads: int, rank_v: int,
                     rank_k: int) -> Dict[str, np.ndarray]:
    """Factors fitted against the attention output: per KV head g, B and the
    group's folded projections from the reduced-rank fit of V.W_g, then P,
    R_enc and R_dec as in fit_factors on the latents V.B.  K, V: calibration
    tokens [n][H_kv][d_h]; W_O: [n_q_heads*d_h][d_model].  Returns fp32 B,
    P, R_enc, R_dec in the library's layout and W_ofT [d_model][n_q_heads*r]
    (fp32; round it to the storage dtype)."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    W_O = np.asarray(W_O, np.float64)
    n, H, D = V.shape
    G = n_q_heads // H
    dm = W_O.shape[1]
    if W_O.shape[0] != n_q_heads * D or n_q_heads % H:
        raise ValueError("W_O must be [n_q_heads * d_h][d_model] with n_q_heads a multiple of n_kv_heads")
    base = fit_factors(K, V, rank_v, rank_k)  # shapes; B, P, R_* replaced below
    W_ofT = np.zeros((dm, n_q_heads * rank_v), np.float32)
    for g in range(H):
        v, k = V[:, g], K[:, g]
        Wg = np.concatenate([W_O[(g * G + i) * D:(g * G + i + 1) * D] for i in range(G)], axis=1)
        U = _leading_right_vectors(v @ Wg, rank_v)  # [G*dm][r]
        B = Wg @ U
        C = U.T                                     # [r][G*dm]
        Z = v @ B
        P, *_ = np.linalg.lstsq(Z, k, rcond=None)
        Re = _leading_right_vectors(k - Z @ P, rank_k)
        base["B"][g], base["P"][g], base["R_enc"][g], base["R_dec"][g] = B, P, Re, Re.T
        for i in range(G):
            h = g * G + i
            W_ofT[:, h * rank_v:(h + 1) * rank_v] = C[:, i * dm:(i + 1) * dm].T
    base["W_ofT"] = W_ofT
    return base


def fit_joint_projection(O: np.ndarray, W_O: np.ndarray, B: np.ndarray) -> np.ndarray:
    """The folded projections of every query head fitted together against the
    layer's whole output (the pages' joint fit across partitions, for a fixed
    latent basis).  O: calibration attention outputs [n][H_q][d_h] (for each
    calibration query, head h's softmax-weighted Values); W_O:
    [H_q*d_h][d_model]; B: [H_kv][d_h][r], head h reading B[h // group].
    Since ẑ_h = o_h.B before rounding, the layer output Σ_h o_h.W_O[h] is
    approximated by Σ_h (o_h.B_g(h)).W_of[h]: linear in all the W_of[h] at
    once, so one least-squares solve over the n calibration rows fits them
    jointly, each head's block knowing every other head's error (heads on
    other GPUs included when O and W_O hold the whole layer; a GPU keeps its
    heads' columns).  Returns W_ofT [d_model][H_q*r] (fp32)."""
    O = np.asarray(O, np.float64)
    W_O = np.asarray(W_O, np.float64)
    B = np.asarray(B, np.float64)
    n, Hq, D = O.shape
    H, _, r = B.shape
    if B.shape[1] != D or Hq % H or W_O.shape[0] != Hq * D:
        raise ValueError("O [n][H_q][d_h], W_O [H_q*d_h][d_model], B [H_kv][d_h][r] with H_q a multiple of H_kv")
    G = Hq // H
    Y = sum(O[:, h] @ W_O[h * D:(h + 1) * D] for h in range(Hq))        # [n][d_model]
    X = np.concatenate([O[:, h] @ B[h // G] for h in range(Hq)], axis=1)  # [n][H_q*r]
    W_of, *_ = np.linalg.lstsq(X, Y, rcond=None)                          # [H_q*r][d_model]
    return np.ascontiguousarray(W_of.T, np.float32)


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
