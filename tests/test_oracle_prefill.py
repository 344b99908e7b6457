"""Pins of the oracle's chunked-prefill attention (CPU only).

Query token t of a chunk sits at position start + t and attends the cached tokens up to and
including its own position (the summary's §3 step 3 read, once per query token). Pins: a cache
held entirely in the exact tail is plain causal attention (torch's scaled_dot_product_attention
with is_causal in fp64); a single-token chunk is the decode; a token's logits are the decode's
logits at its own length, whatever comes later in the chunk.
"""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import oracle as orc
from workloads import synth

from .helpers import value_payload

W = synth.scaled(synth.WORKLOADS["qwen7b_decode"], n_q_heads=4, n_kv_heads=2, batch=2, n_ctx=96, rank=16)


def _cache(w, U, K, V, cap, pieces):
    c = orc.empty_cache(K.shape[0], K.shape[1], cap, w.head_dim, w.rank, 0, 1, key_dtype=1)
    for b in range(K.shape[0]):
        for h in range(K.shape[1]):
            for st, n in pieces:
                orc.write_stream(c, b, h, st, K[b, h, st:st + n], value_payload(V[b, h, st:st + n], w), U[h], 0, 1)
    return c


def _queries(w, B, n_q, seed=3):
    rng = np.random.default_rng(seed)
    return synth.round_to(rng.standard_normal((B, n_q, w.n_q_heads, w.head_dim)).astype(np.float32), "bf16")


def test_all_tail_prefill_is_causal_attention():
    w = W
    U = orc.calibrate(synth.calibration_queries(w, n_cal=64), 2, 16)[0]
    K = synth.stack_streams(w, "keys", 2, 29)
    V = synth.stack_streams(w, "values", 2, 29)
    cache = _cache(w, U, K, V, 32, [(0, 29)])
    q = _queries(w, 2, 29)
    _, out = orc.prefill(cache, q, U, 0)
    g = w.gqa
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)             # [B][Hq][T][d]
    Kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(g, dim=1)     # [B][Hq][T][d]
    Vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(g, dim=1)
    ref = F.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True).permute(0, 2, 1, 3).numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_single_token_chunk_is_the_decode_and_rows_are_causal():
    w = W
    U = orc.calibrate(synth.calibration_queries(w, n_cal=64), 2, 16)[0]
    K = synth.stack_streams(w, "keys", 2, 90)
    V = synth.stack_streams(w, "values", 2, 90)
    cache = _cache(w, U, K, V, 96, [(0, 64), (64, 26)])
    q = _queries(w, 2, 20)
    lg, out = orc.prefill(cache, q, U, 70)
    for t in (0, 7, 19):
        ref_l, ref_o = orc.decode(cache, q[:, t], U, 70 + t + 1, 1.0, 0, 1)
        assert np.array_equal(lg[:, t, :, :71 + t], ref_l)
        assert np.all(lg[:, t, :, 71 + t:] == 0)
        assert np.array_equal(out[:, t], ref_o)
