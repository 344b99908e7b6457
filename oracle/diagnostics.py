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

score_diagnostics() applies these definitions to a packed cache: the cache's corrected logits
(the oracle decode) against the exact scores of reference keys, per (batch row, query head).
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


STATS = ("fisher_var", "kl", "mean_ds", "max_abs_ds", "a2", "entropy")


def score_diagnostics(cache, q, U, n_ctx, kappa, K_ref, V_ref=None, value_mode=0, value_dtype=1):
    """Score-space diagnostics of a packed cache against the keys (and values) it was written
    from, for every (b, query head), over the first n_ctx tokens. Returns f64 [B][Hq][6] in the
    order of STATS:
      fisher_var  Var_p(ds) with p = softmax(s), s_j = q.k_j/sqrt(d) from the reference keys and
                  ds_j = s_hat_j - s_j, s_hat the cache's corrected logits (kappa scales the
                  correction) — the Fisher-weighted score error of §2.1
      kl          KL(p || softmax(s_hat)), by its definition
      mean_ds     E_p[ds] (the softmax-null part of the error)
      max_abs_ds  max_j |ds_j|
      a2          sum_j p_j^2 |v_hat_j - v_j|^2, the A^2 surrogate of §2.2 (NaN without V_ref)
      entropy     -sum_j p_j log p_j of the exact attention
    q: f32 [B][Hq][d]; K_ref, V_ref: f32 [B][Hkv][>= n_ctx][d] (exact widenings of the stored
    dtypes). Query head a reads KV head a // (Hq / Hkv)."""
    from . import oracle as orc
    s_hat, _ = orc.decode(cache, q, U, n_ctx, kappa, value_mode, value_dtype)
    B, Hq, d = q.shape
    Hkv = K_ref.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, len(STATS)), np.float64)
    for b in range(B):
        for h in range(Hkv):
            K = np.asarray(K_ref[b, h, :n_ctx], np.float64)
            dV = None
            if V_ref is not None:
                dV = orc.value_rows(cache, b, h, n_ctx, value_mode, value_dtype) - np.asarray(V_ref[b, h, :n_ctx],
                                                                                           np.float64)
            for a in range(h * g, (h + 1) * g):
                s = scores(q[b, a], K)
                ds = s_hat[b, a] - s
                p = softmax(s)
                out[b, a] = (fisher_variance(p, ds), kl(p, softmax(s_hat[b, a])), float(p @ ds),
                             float(np.max(np.abs(ds))), np.nan if dV is None else a2_surrogate(p, dV),
                             float(-np.sum(p[p > 0] * np.log(p[p > 0]))))
    return out


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
