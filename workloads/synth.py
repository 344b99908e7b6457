"""Seeded synthetic workloads shaped like the HeadQ evaluation models.

This module holds none of the method's arithmetic: it only draws keys, values and queries with
the shapes and distributions of the five workloads below, so that the GPU library and the CPU
oracle can be fed the very same arrays. The pages evaluate on WikiText-103 with six trained
models; neither the data nor the weights are available, so these draws stand in for them with
the models' attention shapes (head counts, head_dim, GQA ratio, context, batch).

Recipe (same for every workload, per (batch b, KV head h) stream, each stream seeded on its own
so any slice can be regenerated without the rest):
  keys    pre-RoPE N(0,1); on a seed-chosen set of outlier channels per KV head (4 or 8) the
          channel is multiplied by exp(N(0,1)); rotate-half RoPE with base 10000 at positions
          0..T-1; rounded to the key dtype.
  values  N(0,1), rounded to the value dtype.
  calibration queries  per query head a fixed A in R^{d x 8} with N(0,1) entries,
          q = A z + 0.1 eps (z ~ N(0, I_8), eps ~ N(0, I_d)), RoPE at positions 0..n_cal-1.
  decode queries  the same per-head distribution from a separate seed stream, RoPE at the
          decode position n_ctx.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# seed-stream identifiers
_KEYS, _VALUES, _OUTLIERS, _QPROJ, _QCAL, _QDEC = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    head_dim: int
    n_q_heads: int
    n_kv_heads: int
    batch: int
    n_ctx: int
    rank: int
    n_outliers: int
    key_dtype: str        # "f32" | "bf16"
    value_dtype: str      # "f32" | "bf16"
    value_mode: str       # "dense" | "q2"
    query_dtype: str      # "f32" | "bf16"
    layers: int = 1
    n_cal: int = 512
    base_bits: int = 2
    side_bits: int = 4
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    "tiny": Workload("tiny", 1000, 64, 1, 1, 1, 256, 8, 4, "f32", "f32", "dense", "f32"),
    "tinyllama_decode": Workload("tinyllama_decode", 1001, 64, 32, 4, 16, 4096, 16, 4, "bf16", "bf16",
                                 "dense", "bf16", layers=22),
    "qwen7b_decode": Workload("qwen7b_decode", 1002, 128, 28, 4, 32, 16384, 16, 8, "bf16", "bf16", "dense",
                              "bf16"),
    "append_prefill": Workload("append_prefill", 1003, 128, 8, 8, 1, 32768, 32, 8, "bf16", "bf16", "dense",
                               "bf16"),
    "qwen14b_fullkv": Workload("qwen14b_fullkv", 1004, 128, 40, 8, 64, 32768, 16, 8, "bf16", "bf16", "q2",
                               "bf16"),
}


def _rng(seed: int, *path: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, *path]))


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round f32 values to `dtype` and widen back exactly (f32 result)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        # round to nearest even on the upper 16 bits (inputs here are finite)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return (u.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def rope(x: np.ndarray, positions: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate-half rotary embedding: pairs (i, i + d/2), angle pos * base^(-2i/d)."""
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = positions.astype(np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half].astype(np.float64), x[..., half:].astype(np.float64)
    out = np.empty(x.shape, np.float64)
    out[..., :half] = x1 * c - x2 * s
    out[..., half:] = x2 * c + x1 * s
    return out.astype(np.float32)


def outlier_scales(w: Workload, h: int) -> np.ndarray:
    g = _rng(w.seed, _OUTLIERS, h)
    scales = np.ones(w.head_dim, np.float64)
    ch = g.choice(w.head_dim, size=w.n_outliers, replace=False)
    scales[ch] = np.exp(g.standard_normal(w.n_outliers))
    return scales


def keys(w: Workload, b: int, h: int, T: int | None = None, start: int = 0) -> np.ndarray:
    """Post-RoPE keys of stream (b, h), tokens [start, start+T), widened to f32 [T][d]."""
    T = w.n_ctx if T is None else T
    g = _rng(w.seed, _KEYS, b, h)
    full = g.standard_normal((start + T, w.head_dim), dtype=np.float32)[start:]
    full = full * outlier_scales(w, h)[None, :].astype(np.float32)
    return round_to(rope(full, np.arange(start, start + T)), w.key_dtype)


def values(w: Workload, b: int, h: int, T: int | None = None, start: int = 0) -> np.ndarray:
    T = w.n_ctx if T is None else T
    g = _rng(w.seed, _VALUES, b, h)
    full = g.standard_normal((start + T, w.head_dim), dtype=np.float32)[start:]
    return round_to(full, w.value_dtype)


def _qproj(w: Workload, hq: int) -> np.ndarray:
    return _rng(w.seed, _QPROJ, hq).standard_normal((w.head_dim, 8))


def calibration_queries(w: Workload, n_cal: int | None = None) -> np.ndarray:
    """f32 [Hq][n_cal][d] post-RoPE calibration queries (low-rank(8) Gaussian + 0.1 noise)."""
    n = w.n_cal if n_cal is None else n_cal
    out = np.empty((w.n_q_heads, n, w.head_dim), np.float32)
    for hq in range(w.n_q_heads):
        g = _rng(w.seed, _QCAL, hq)
        z = g.standard_normal((n, 8))
        eps = g.standard_normal((n, w.head_dim))
        q = z @ _qproj(w, hq).T + 0.1 * eps
        out[hq] = rope(q.astype(np.float32), np.arange(n))
    return out


def decode_queries(w: Workload, position: int | None = None, batch: int | None = None,
                   stream: int = 0) -> np.ndarray:
    """f32 [B][Hq][d] decode queries (held-out draws of the calibration distribution), rounded to
    the query dtype. `stream` selects independent draws (e.g. one per layer)."""
    pos = w.n_ctx if position is None else position
    B = w.batch if batch is None else batch
    out = np.empty((B, w.n_q_heads, w.head_dim), np.float32)
    for hq in range(w.n_q_heads):
        g = _rng(w.seed, _QDEC, hq, stream)
        z = g.standard_normal((B, 8))
        eps = g.standard_normal((B, w.head_dim))
        q = z @ _qproj(w, hq).T + 0.1 * eps
        out[:, hq] = rope(q.astype(np.float32), np.full(B, pos))
    return round_to(out, w.query_dtype)


def scaled(w: Workload, **changes) -> Workload:
    """A copy of `w` with some fields changed (smaller parity cases of the same recipe)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(changes)
    return Workload(**d)


def stack_streams(w: Workload, kind: str, batch: int | None = None, T: int | None = None,
                  workers: int = 8) -> np.ndarray:
    """All (b, h) streams of `kind` ("keys" or "values") as f32 [B][Hkv][T][d], generated in a
    thread pool (each stream is seeded on its own, so the result does not depend on `workers`)."""
    from concurrent.futures import ThreadPoolExecutor

    B = w.batch if batch is None else batch
    T = w.n_ctx if T is None else T
    fn = keys if kind == "keys" else values
    out = np.empty((B, w.n_kv_heads, T, w.head_dim), np.float32)

    def one(bh):
        b, h = divmod(bh, w.n_kv_heads)
        out[b, h] = fn(w, b, h, T)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(B * w.n_kv_heads)))
    return out
