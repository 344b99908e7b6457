"""Pins of the oracle's chunked-prefill attention (CPU only).

Query token t of a chunk sits at position start + t and attends the cached tokens up to and
including its own position (the summary's §3 step 3 read, once per query token), in the cache
as it stands after the chunk's append (whole groups packed, the unfinished group exact). Pins: a
cache held entirely in the exact tail is plain causal attention (torch's
scaled_dot_product_attention with is_causal in fp64); so is a cache whose keys lie on the base
grid (zero quantization error), with query positions inside whole packed groups; the chunk's
last token is the decode over the whole cache; every token's logits are the whole-cache decode
logits cut at its position.
"""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import oracle as orc
from workloads import synth

from .helpers import value_payload
from .test_oracle_method import _on_grid_keys

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


def test_rows_are_the_whole_cache_decode_cut_at_their_position():
    w = W
    U = orc.calibrate(synth.calibration_queries(w, n_cal=64), 2, 16)[0]
    K = synth.stack_streams(w, "keys", 2, 90)
    V = synth.stack_streams(w, "values", 2, 90)
    cache = _cache(w, U, K, V, 96, [(0, 50), (50, 40)])  # groups 0, 1 packed; 64..89 in the tail
    q = _queries(w, 2, 45)                               # positions 45 .. 89: inside group 1, then the tail
    lg, out = orc.prefill(cache, q, U, 45)
    for t in (0, 18, 19, 44):
        ref_l, ref_o = orc.decode(cache, q[:, t], U, 90, 1.0, 0, 1)
        assert np.array_equal(lg[:, t, :, :46 + t], ref_l[:, :, :46 + t])
        assert np.all(lg[:, t, :, 46 + t:] == 0)
    ref_l, ref_o = orc.decode(cache, q[:, 44], U, 90, 1.0, 0, 1)
    assert np.allclose(out[:, 44], ref_o, rtol=0, atol=1e-13)


def test_keys_on_the_grid_give_causal_attention_inside_packed_groups():
    w = synth.scaled(W, rank=0)
    rng = np.random.default_rng(9)
    K = np.stack([np.stack([_on_grid_keys(rng, 96, 128) for _ in range(2)]) for _ in range(2)])
    K = synth.round_to(K, "bf16")  # the grid values are dyadic and survive bf16 rounding
    V = synth.stack_streams(w, "values", 2, 96)
    c = orc.empty_cache(2, 2, 96, 128, 0, 0, 1, key_dtype=1)
    for b in range(2):
        for h in range(2):
            orc.write_stream(c, b, h, 0, K[b, h], value_payload(V[b, h], w), None, 0, 1)
    q = _queries(w, 2, 96)
    _, out = orc.prefill(c, q, None, 0)
    g = w.gqa
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    Kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(g, dim=1)
    Vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(g, dim=1)
    ref = F.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True).permute(0, 2, 1, 3).numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
