"""Score-space diagnostics of the HeadQ pages, in plain fp64 numpy — TEST INFRASTRUCTURE ONLY.

Sources ("Technische Samenvatting: HeadQ ...", the Dutch technical summary):
  §2.1  a key error dk_j reaches the model only through the score ds_j = q.dk_j / sqrt(d);
        a shift shared by all tokens is softmax-null; the KL between the original and the
        perturbed attention is locally a Fisher-weighted variance of the score errors (its
        Eq. 6, not printed; reading: KL ~ 1/2 ds^T (diag p - p p^T) ds).
  §2.2  for fixed attention p the readout error is dO = sum_j p_j dv_j; the A^2 surrogate
        weighs each token's value distortion by p_j^2.
  §4    controls: null-space intervention with a non-equivariant fixed-grid quantizer,
        same-budget counterexamples, query-PCA versus random bases, wrong-sign correction.
"""
from __future__ import annotations

import numpy as np


def softmax(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def scores(q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """s_j = q.k_j / sqrt(d) (§2.1). q: [d], K: [T][d]."""
    q = np.asarray(q, np.float64)
    return np.asarray(K, np.float64) @ q / np.sqrt(q.shape[-1])


def fisher_matrix(p: np.ndarray) -> np.ndarray:
    """Fisher information of the softmax in score coordinates: diag(p) - p p^T."""
    p = np.asarray(p, np.float64)
    return np.diag(p) - np.outer(p, p)


def fisher_variance(p: np.ndarray, ds: np.ndarray) -> float:
    """Var_p(ds) = sum p ds^2 - (sum p ds)^2 = ds^T F ds (§2.1, Eq. 6 reading)."""
    p = np.asarray(p, np.float64)
    ds = np.asarray(ds, np.float64)
    m = float(p @ ds)
    return float(p @ (ds * ds) - m * m)


def kl(p: np.ndarray, p_hat: np.ndarray) -> float:
    """KL(p || p_hat) computed directly."""
    p = np.asarray(p, np.float64)
    p_hat = np.asarray(p_hat, np.float64)
    mask = p > 0
    return float(np.sum(p[mask] * (np.log(p[mask]) - np.log(p_hat[mask]))))


def readout_error(p: np.ndarray, dV: np.ndarray) -> np.ndarray:
    """dO = sum_j p_j dv_j for fixed attention p (§2.2)."""
    return np.asarray(p, np.float64) @ np.asarray(dV, np.float64)


def a2_surrogate(p: np.ndarray, dV: np.ndarray) -> float:
    """sum_j p_j^2 |dv_j|^2: the A^2-weighted token distortion (§2.2)."""
    p = np.asarray(p, np.float64)
    dV = np.asarray(dV, np.float64)
    return float(np.sum(p * p * np.sum(dV * dV, axis=-1)))


def fixed_grid_quantize(K: np.ndarray, step: float, levels: int) -> np.ndarray:
    """A toy non-equivariant quantizer: symmetric fixed grid round(k/step)*step clamped to
    +-levels*step, identical for every token and channel (used for the §4 null-space control)."""
    q = np.clip(np.rint(np.asarray(K, np.float64) / step), -levels, levels)
    return q * step


def minmax_quantize(K: np.ndarray, bits: int = 2, group: int = 32) -> np.ndarray:
    """A plain per-channel asymmetric min/max quantizer over token groups, in fp64 (the
    equivariant counterpart of the toy fixed grid; no storage rounding)."""
    K = np.asarray(K, np.float64)
    T, d = K.shape
    L = (1 << bits) - 1
    out = np.empty_like(K)
    for g0 in range(0, T, group):
        blk = K[g0:g0 + group]
        lo, hi = blk.min(axis=0), blk.max(axis=0)
        s = (hi - lo) / L
        inv = np.where(s > 0, 1.0 / np.where(s > 0, s, 1.0), 0.0)
        c = np.clip(np.rint((blk - lo) * inv), 0, L)
        out[g0:g0 + group] = c * s + lo
    return out


def spearman(x: np.ndarray, y: np.ndarray) -> float:
    """Spearman rank correlation (average ranks for ties)."""
    def ranks(a):
        a = np.asarray(a, np.float64)
        order = np.argsort(a, kind="mergesort")
        r = np.empty(len(a), np.float64)
        r[order] = np.arange(len(a), dtype=np.float64)
        # average ties
        vals, inv, counts = np.unique(a, return_inverse=True, return_counts=True)
        sums = np.zeros(len(vals))
        np.add.at(sums, inv, r)
        return (sums / counts)[inv]
    rx, ry = ranks(x), ranks(y)
    rx -= rx.mean()
    ry -= ry.mean()
    return float(rx @ ry / np.sqrt((rx @ rx) * (ry @ ry)))
