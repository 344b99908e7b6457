"""Oracle pins for token-granular cache writes (the dense tail of the unfinished last group).

A cache write may append any number of tokens (the summary's §3 step 2 is a per-token cache
write); whole 32-token groups are encoded, the tokens of the unfinished last group stay exact in a
dense tail, and decode reads them with exact keys and values. The pins: a context held entirely in
the tail is exact attention (torch's scaled_dot_product_attention in fp64); appending one token at
a time produces the same packed groups as one aligned write; a mixed context's logits are the
aligned cache's logits followed by the exact q.k/sqrt(d) of the tail tokens, read out with the
exact softmax.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle as orc
from workloads import synth

from .helpers import value_payload

W = synth.scaled(synth.WORKLOADS["qwen7b_decode"], n_q_heads=4, n_kv_heads=2, batch=2, n_ctx=128, rank=16)
PACKED = ("kcode", "kmeta", "scode", "ssc", "v", "vcode", "vmeta")


def _sdpa(q, K, V, g):
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    Kt = torch.from_numpy(np.asarray(K, np.float64)).repeat_interleave(g, dim=0)[None]
    Vt = torch.from_numpy(np.asarray(V, np.float64)).repeat_interleave(g, dim=0)[None]
    return F.scaled_dot_product_attention(qt, Kt, Vt)[0, :, 0, :].numpy()


def _streams(w, T):
    return {(b, h): (synth.keys(w, b, h, T), synth.values(w, b, h, T)) for b in range(w.batch) for h in
            range(w.n_kv_heads)}


def _cache(w, U, cap):
    return orc.empty_cache(w.batch, w.n_kv_heads, cap, w.head_dim, 0 if U is None else U.shape[2],
                           0 if w.value_mode == "dense" else 1, 0 if w.value_dtype == "f32" else 1,
                           key_dtype=0 if w.key_dtype == "f32" else 1)


def _append(cache, w, U, kv, pieces):
    vm = 0 if w.value_mode == "dense" else 1
    vd = 0 if w.value_dtype == "f32" else 1
    for (b, h), (k, v) in kv.items():
        for start, n in pieces:
            orc.write_stream(cache, b, h, start, k[start:start + n], value_payload(v[start:start + n], w),
                             None if U is None else U[h], vm, vd)


def _U(w):
    return orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0]


@pytest.mark.parametrize("n_ctx", [1, 7, 31])
def test_context_inside_the_tail_is_exact_attention(n_ctx):
    w = W
    U = _U(w)
    kv = _streams(w, n_ctx)
    cache = _cache(w, U, 64)
    _append(cache, w, U, kv, [(i, 1) for i in range(n_ctx)])
    q = synth.decode_queries(w, position=n_ctx)
    lg, out = orc.decode(cache, q, U, n_ctx, 1.0, 0, 1)
    for b in range(w.batch):
        K = np.stack([kv[(b, h)][0] for h in range(w.n_kv_heads)])
        V = np.stack([kv[(b, h)][1] for h in range(w.n_kv_heads)])
        assert np.allclose(out[b], _sdpa(q[b], K, V, w.gqa), rtol=0, atol=1e-12)
        exact = np.einsum("hd,htd->ht", q[b].astype(np.float64), np.repeat(K, w.gqa, axis=0)) / np.sqrt(128.0)
        assert np.allclose(lg[b], exact, rtol=0, atol=1e-12)


@pytest.mark.parametrize("wname", ["qwen7b_decode", "qwen14b_fullkv"])
def test_token_by_token_append_equals_aligned_write(wname):
    w = synth.scaled(synth.WORKLOADS[wname], n_q_heads=4, n_kv_heads=2, batch=1, n_ctx=96)
    U = _U(w)
    kv = _streams(w, 96)
    one = _cache(w, U, 128)
    _append(one, w, U, kv, [(i, 1) for i in range(96)])
    mixed = _cache(w, U, 128)
    _append(mixed, w, U, kv, [(0, 40), (40, 1), (41, 19), (60, 36)])  # tail reads, whole groups, new tail
    ref = _cache(w, U, 128)
    _append(ref, w, U, kv, [(0, 96)])
    for name in PACKED:
        if name in ref:
            assert np.array_equal(one[name], ref[name]), name
            assert np.array_equal(mixed[name], ref[name]), name


def test_partial_last_group_kept_exact_in_tail():
    w = W
    U = _U(w)
    kv = _streams(w, 100)
    cache = _cache(w, U, 128)
    _append(cache, w, U, kv, [(0, 40), (40, 60)])  # groups 0..2 whole, tokens 96..99 in the tail
    for (b, h), (k, v) in kv.items():
        assert np.array_equal(orc.bf16_bits_to_f32(cache["ktail"][b, h, :4]), k[96:100])
        assert np.array_equal(orc.bf16_bits_to_f32(cache["vtail"][b, h, :4]), v[96:100])


@pytest.mark.parametrize("wname,n_ctx", [("qwen7b_decode", 77), ("qwen7b_decode", 96 + 31)])
def test_mixed_context_logits_and_readout(wname, n_ctx):
    w = synth.scaled(synth.WORKLOADS[wname], n_q_heads=4, n_kv_heads=2, batch=1, n_ctx=n_ctx)
    U = _U(w)
    kv = _streams(w, n_ctx)
    n_full = n_ctx // 32 * 32
    cache = _cache(w, U, 128)
    _append(cache, w, U, kv, [(0, n_full)] + [(i, 1) for i in range(n_full, n_ctx)])
    aligned = _cache(w, U, 128)
    _append(aligned, w, U, kv, [(0, n_full)])
    q = synth.decode_queries(w, position=n_ctx)
    lg, out = orc.decode(cache, q, U, n_ctx, 1.0, 0, 1)
    lg_full, _ = orc.decode(aligned, q, U, n_full, 1.0, 0, 1)
    K = np.stack([kv[(0, h)][0] for h in range(2)])
    V = np.stack([kv[(0, h)][1] for h in range(2)])
    Kr = np.repeat(K, w.gqa, axis=0)
    Vr = np.repeat(V, w.gqa, axis=0).astype(np.float64)
    tail = np.einsum("hd,htd->ht", q[0].astype(np.float64), Kr[:, n_full:]) / np.sqrt(128.0)
    assert np.array_equal(lg[0, :, :n_full], lg_full[0])
    assert np.allclose(lg[0, :, n_full:], tail, rtol=0, atol=1e-12)
    p = np.exp(lg[0] - lg[0].max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    # dense bf16 values are stored exactly, so the readout is the plain softmax-weighted sum
    assert np.allclose(out[0], np.einsum("ht,htd->hd", p, Vr), rtol=0, atol=1e-12)


def test_decode_rejects_a_partial_group_without_tails():
    w = W
    cache = orc.empty_cache(1, 2, 64, 128, 0, 0, 1)  # no tails
    with pytest.raises(ValueError):
        orc.decode(cache, np.zeros((1, 4, 128), np.float32), None, 40, 1.0, 0, 1)
