"""Shared test helpers: building oracle caches from the seeded workloads."""
from __future__ import annotations

import numpy as np

from oracle import oracle as orc
from workloads import synth

VDT = {"f32": 0, "bf16": 1}
VMODE = {"dense": 0, "q2": 1}


def value_payload(v_f32: np.ndarray, w: synth.Workload):
    """Values in the form the oracle packer takes: f32 array (f32 dtype or 2-bit mode) or the
    bf16 bit patterns (exact, the generator already rounded them)."""
    if w.value_mode == "q2" or w.value_dtype == "f32":
        return np.ascontiguousarray(v_f32, np.float32)
    return (np.ascontiguousarray(v_f32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def oracle_cache(w: synth.Workload, U: np.ndarray | None, batch: int | None = None, n_tok: int | None = None,
                 cap: int | None = None, bits: int | None = None, kv=None):
    """Encode the workload's streams with the oracle. Returns (cache, per-stream encodes).
    kv: optional dict {(b, h): (k, v)} overriding the generator."""
    B = w.batch if batch is None else batch
    T = w.n_ctx if n_tok is None else n_tok
    cap = T if cap is None else cap
    r = 0 if U is None else U.shape[2]
    cache = orc.empty_cache(B, w.n_kv_heads, cap, w.head_dim, r, VMODE[w.value_mode], VDT[w.value_dtype],
                            base_bits=w.base_bits if bits is None else bits)
    encs = {}
    for b in range(B):
        for h in range(w.n_kv_heads):
            if kv is not None:
                k, v = kv[(b, h)]
            else:
                k, v = synth.keys(w, b, h, T), synth.values(w, b, h, T)
            encs[(b, h)] = orc.write_stream(cache, b, h, 0, k, value_payload(v, w), None if U is None else U[h],
                                            VMODE[w.value_mode], VDT[w.value_dtype],
                                            bits=w.base_bits if bits is None else bits, side_bits=w.side_bits)
    return cache, encs
