"""Pins of the oracle's score-space diagnostics of a packed cache (CPU only).

score_diagnostics() composes the oracle decode (the cache's corrected logits) with the §2.1/§2.2
definitions of "Technische Samenvatting: HeadQ ..." (Fisher variance of the score error, KL of
the attention, the A^2 value surrogate). These tests rebuild the score errors along a path that
never reads the packed cache — the encoder's own codes, steps, zeros and side codes, dequantized
here — and check the composition against scipy's relative entropy and entropy routines; plus
the special cases the definitions fix: keys on the base grid give zero score error, kappa = 0
equals a cache without side code, and dense values stored exactly give A^2 = 0.
"""
import numpy as np
import pytest
from scipy import special, stats

from oracle import diagnostics as dg
from oracle import oracle as orc
from workloads import synth

from .helpers import VDT, VMODE, value_payload
from .test_oracle_method import _on_grid_keys

W = synth.WORKLOADS


def _f16(x):
    return orc.f16_bits_to_f32(x).astype(np.float64)


def _build(w, U, K, V, n_ctx):
    """Oracle cache of K/V [B][Hkv][n_ctx][d]: whole groups in one write, the rest into the tails.
    Returns (cache, encoder outputs per stream)."""
    B, H = K.shape[:2]
    n_full = n_ctx // 32 * 32
    cap = (n_ctx + 31) // 32 * 32
    c = orc.empty_cache(B, H, cap, w.head_dim, 0 if U is None else U.shape[2], VMODE[w.value_mode],
                        VDT[w.value_dtype], key_dtype=VDT[w.key_dtype], base_bits=w.base_bits)
    enc = {}
    for b in range(B):
        for h in range(H):
            Uh = None if U is None else U[h]
            vm, vd = VMODE[w.value_mode], VDT[w.value_dtype]
            if n_full:
                enc[(b, h)] = orc.write_stream(c, b, h, 0, K[b, h, :n_full], value_payload(V[b, h, :n_full], w), Uh,
                                               vm, vd, bits=w.base_bits)
            if n_ctx > n_full:
                orc.write_stream(c, b, h, n_full, K[b, h, n_full:n_ctx], value_payload(V[b, h, n_full:n_ctx], w), Uh,
                                 vm, vd, bits=w.base_bits)
    return c


def _independent(w, U, K, V, q, n_ctx, kappa):
    """The six statistics from the encoder's outputs (no cache unpacking) and scipy."""
    B, H = K.shape[:2]
    Hq, d = q.shape[1], q.shape[2]
    g = Hq // H
    n_full = n_ctx // 32 * 32
    out = np.zeros((B, Hq, 6))
    for b in range(B):
        for h in range(H):
            k = K[b, h, :n_ctx].astype(np.float64)
            e = orc.encode_keys(K[b, h, :n_full], None if U is None else U[h]) if n_full else None
            k_hat = k.copy()                      # tail tokens are exact
            zhat = None
            if n_full:
                gi = np.arange(n_full) // 32
                k_hat[:n_full] = e["codes"].astype(np.float64) * _f16(e["scale"])[gi] + _f16(e["zero"])[gi]
                if U is not None:
                    zhat = _f16(e["sigma"])[:, None] * e["zc"].astype(np.float64)
            v = V[b, h, :n_ctx].astype(np.float64)
            v_hat = v.copy()
            if w.value_mode == "q2" and n_full:
                vq = orc.quantize_values(V[b, h, :n_full])
                ci = np.arange(d) // 32
                v_hat[:n_full] = vq["codes"] * _f16(vq["scale"])[:, ci] + _f16(vq["zero"])[:, ci]
            for a in range(h * g, (h + 1) * g):
                qa = q[b, a].astype(np.float64)
                s = k @ qa / np.sqrt(d)
                s_hat = k_hat @ qa / np.sqrt(d)
                if zhat is not None:
                    qu = U[h].astype(np.float64).T @ qa
                    s_hat[:n_full] += kappa * (zhat @ qu) / np.sqrt(d)
                ds = s_hat - s
                p = special.softmax(s)
                out[b, a] = (p @ (ds * ds) - (p @ ds) ** 2, special.rel_entr(p, special.softmax(s_hat)).sum(),
                             p @ ds, np.abs(ds).max(), np.sum(p * p * np.sum((v_hat - v) ** 2, axis=1)),
                             stats.entropy(p))
    return out


def _inputs(w, B, n_ctx, seed=0):
    K = synth.stack_streams(w, "keys", B, n_ctx)
    V = synth.stack_streams(w, "values", B, n_ctx)
    q = synth.decode_queries(w, position=n_ctx, batch=B)
    return K, V, q


def _close(a, b, rtol=1e-9, atol=1e-13):
    assert np.allclose(a, b, rtol=rtol, atol=atol), np.max(np.abs(a - b))


@pytest.mark.parametrize("wname,n_ctx,kappa", [("tiny", 96, 1.0), ("tiny", 96 + 13, -1.0),
                                               ("qwen7b_decode", 64 + 5, 1.0), ("qwen14b_fullkv", 128, 1.0),
                                               ("qwen14b_fullkv", 64 + 31, 0.5)])
def test_diagnostics_match_the_encoder_path(wname, n_ctx, kappa):
    w = synth.scaled(W[wname], n_q_heads=4, n_kv_heads=2, batch=2, rank=min(W[wname].rank, 8))
    U = orc.calibrate(synth.calibration_queries(w, n_cal=64), w.n_kv_heads, w.rank)[0]
    K, V, q = _inputs(w, 2, n_ctx)
    cache = _build(w, U, K, V, n_ctx)
    got = dg.score_diagnostics(cache, q, U, n_ctx, kappa, K, V, VMODE[w.value_mode], VDT[w.value_dtype])
    ref = _independent(w, U, K, V, q, n_ctx, kappa)
    _close(got, ref)
    assert np.all(got[..., 0] > 0) and np.all(got[..., 1] > 0)   # real quantization error is visible
    if w.value_mode == "dense":
        assert np.all(got[..., 4] == 0.0)                        # dense values are stored exactly


def test_keys_on_the_base_grid_have_zero_score_error():
    w = synth.scaled(W["tiny"], n_q_heads=2, n_kv_heads=1, batch=1, rank=8)
    rng = np.random.default_rng(21)
    K = _on_grid_keys(rng, 64, 64)[None, None]
    V = rng.standard_normal((1, 1, 64, 64)).astype(np.float32)
    q = rng.standard_normal((1, 2, 64)).astype(np.float32)
    U = orc.calibrate(synth.calibration_queries(w, n_cal=64), 1, 8)[0]
    got = dg.score_diagnostics(_build(w, U, K, V, 64), q, U, 64, 1.0, K, V, 0, 0)
    assert np.all(np.abs(got[..., :4]) < 1e-12)
    for a in range(2):
        assert np.isclose(got[0, a, 5], stats.entropy(special.softmax(K[0, 0].astype(np.float64) @ q[0, a] / 8.0)))


def test_kappa_zero_equals_a_cache_without_side_code():
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=4, n_kv_heads=2, batch=1, rank=16)
    U = orc.calibrate(synth.calibration_queries(w, n_cal=64), 2, 16)[0]
    K, V, q = _inputs(w, 1, 96)
    with_side = dg.score_diagnostics(_build(w, U, K, V, 96), q, U, 96, 0.0, K, V, 0, 1)
    w0 = synth.scaled(w, rank=0)
    base = dg.score_diagnostics(_build(w0, None, K, V, 96), q, None, 96, 1.0, K, V, 0, 1)
    _close(with_side, base, rtol=1e-12, atol=1e-15)
    corrected = dg.score_diagnostics(_build(w, U, K, V, 96), q, U, 96, 1.0, K, V, 0, 1)
    assert np.all(corrected[..., 0] < with_side[..., 0])          # the correction removes score error


def test_without_reference_values_a2_is_nan():
    w = synth.scaled(W["tiny"], batch=1)
    U = orc.calibrate(synth.calibration_queries(w, n_cal=64), 1, w.rank)[0]
    K, V, q = _inputs(w, 1, 64)
    got = dg.score_diagnostics(_build(w, U, K, V, 64), q, U, 64, 1.0, K, None, 0, 0)
    assert np.all(np.isnan(got[..., 4])) and np.all(np.isfinite(np.delete(got, 4, axis=-1)))
