"""GPU parity of headq_score_diagnostics against the oracle's score_diagnostics.

The library computes, per (b, query head), the Fisher variance of the score error, the KL of the
attention, the mean and largest score error, the A^2 value surrogate and the entropy of the exact
attention (Technische Samenvatting §2.1/§2.2), all in f64; the oracle applies the same
definitions in fp64 numpy to its own decode of the same cache bytes. Both are f64 evaluations of
one definition, differing only in summation order and in the score error being taken from the
key error (library) or as a difference of two logits (oracle), so the bar is a relative 1e-9 with
an absolute floor of 1e-12 (the oracle's logit difference carries ~1e-15 of rounding).
"""
import numpy as np
import pytest

from oracle import diagnostics as dg
from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import gpu_cache, say, to_device
from .helpers import VDT, VMODE
from .test_oracle_diagnostics import _build

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def check_stats(got, ref, what=""):
    """|gpu - oracle| <= 1e-9 |oracle| + 1e-12, NaN where the oracle has NaN."""
    got = np.asarray(got, np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), what
    err = np.abs(got - ref)[~nan]
    tol = (1e-9 * np.abs(ref) + 1e-12)[~nan]
    worst = np.argmax(err / tol)
    assert np.all(err <= tol), f"{what}: stat error {err[worst]:.3e} vs tolerance {tol[worst]:.3e}"


def _run(w, B, n_ctx, kappa=1.0, with_values=True, n_splits=0, cap=None):
    say("diagnostics", w.name, f"B={B} n_ctx={n_ctx} d={w.head_dim} r={w.rank} g={w.gqa}",
        f"v={w.value_mode}/{w.value_dtype} k={w.key_dtype} kappa={kappa} values={with_values} splits={n_splits}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0] if w.rank else None
    n_full = n_ctx // 32 * 32
    pieces = [p for p in [(0, n_full), (n_full, n_ctx - n_full)] if p[1]]
    cap = cap or (n_ctx + 31) // 32 * 32
    dc, K, V = gpu_cache(w, U, B, n_ctx, cap, pieces=pieces)
    q = synth.decode_queries(w, position=n_ctx, batch=B)
    kd = to_device(K, w.key_dtype)
    vd = to_device(V, w.value_dtype) if with_values else None
    got = dc.score_diagnostics(to_device(q, w.query_dtype), kd, vd, n_ctx, corr_scale=kappa,
                               n_splits=n_splits).cpu().numpy()
    oc = _build(w, U, K, V, n_ctx)
    ref = dg.score_diagnostics(oc, q, U, n_ctx, kappa, K, V if with_values else None, VMODE[w.value_mode],
                               VDT[w.value_dtype])
    check_stats(got, ref, w.name)
    return got


def test_qwen7b_shape_dense_values_ragged_tail():
    got = _run(synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2), 2, 200)
    assert np.all(got[..., 4] == 0.0)  # dense bf16 values are stored exactly


def test_fullkv_two_bit_values_both_signs():
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2)
    plus = _run(w, 2, 160, kappa=1.0)
    minus = _run(w, 2, 160, kappa=-1.0)
    # the wrong-sign control raises the Fisher variance (on average over heads: a head whose
    # correction is uncorrelated with its base error may go either way)
    assert minus[..., 0].mean() > plus[..., 0].mean()


def test_tinyllama_shape_d64_eight_heads():
    _run(synth.scaled(W["tinyllama_decode"], n_q_heads=16, n_kv_heads=2), 2, 96 + 31)


def test_tiny_f32_keys_and_values():
    _run(W["tiny"], 2, 256)


def test_sixteen_heads_rank32_kappa0():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=16, n_kv_heads=1, rank=32), 1, 128, kappa=0.0)


def test_rank0_cache():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1, rank=0), 2, 64 + 9)


def test_without_reference_values():
    got = _run(synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1), 1, 96, with_values=False)
    assert np.all(np.isnan(got[..., 4]))


@pytest.mark.parametrize("splits", [1, 3, 5])
def test_split_counts(splits):
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1), 1, 320, n_splits=splits)


def test_context_shorter_than_one_chunk_in_a_larger_cache():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1), 1, 5, cap=256)


def test_full_size_qwen7b_sampled_streams():
    """Qwen2.5-7B-shaped cache at full size (B 32, Hkv 4, 16384 tokens) in the benchmark's launch
    configuration; the oracle recomputes a few (b, h) streams from the generator."""
    import torch
    w = W["qwen7b_decode"]
    say("diagnostics-fullsize", w.name, f"B={w.batch} T={w.n_ctx}")
    U = orc.calibrate(synth.calibration_queries(w), w.n_kv_heads, w.rank)[0]
    dc, K, V = gpu_cache(w, U)
    q = synth.decode_queries(w)
    got = dc.score_diagnostics(to_device(q, w.query_dtype), to_device(K, w.key_dtype), to_device(V, w.value_dtype),
                               w.n_ctx).cpu().numpy()
    torch.cuda.synchronize()
    g = w.gqa
    for b, h in [(0, 0), (31, 3), (17, 2)]:
        wb = synth.scaled(w, batch=1, n_kv_heads=1, n_q_heads=g)
        Kb, Vb = K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1]
        oc = _build(wb, U[h:h + 1], Kb, Vb, w.n_ctx)
        heads = list(range(h * g, (h + 1) * g))
        ref = dg.score_diagnostics(oc, q[b:b + 1, heads], U[h:h + 1], w.n_ctx, 1.0, Kb, Vb, 0, 1)
        check_stats(got[b:b + 1, heads], ref, f"stream {(b, h)}")
