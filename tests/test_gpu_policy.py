"""GPU parity of the A^2 value policy (value_protect = P > 0, 2-bit values).

The append's choice of corrected tokens and their bfloat16 corrections must equal the oracle's
bit for bit (a discrete decision both sides take in the same f32/f64 arithmetic), and the decode,
which adds p_t * correction_t for the chosen tokens, must meet the decode tolerances against the
oracle's fp64 decode of its own cache. Cases: one and two corrected tokens, d = 64 and 128, one
group per matrix product (g = 16) and two groups sharing the columns (g <= 8), dense tails, splits,
the two-groups-per-workgroup append of long writes, paged caches; the chunked prefill and the
score-space diagnostics (A^2 with the corrections).
"""
import numpy as np
import pytest

from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import check_logits, check_out, compare_cache, decode_gpu, gpu_cache, say, to_device
from .helpers import VDT, VMODE, value_payload

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _direction(w, seed=3):
    """The mean calibration query plus a seeded offset, so that the power-of-two weights spread
    over several exponents (any direction is a valid input)."""
    a = orc.mean_query(synth.calibration_queries(w, n_cal=64), w.n_kv_heads)
    rng = np.random.default_rng(seed)
    return (a + 0.5 * rng.standard_normal(a.shape)).astype(np.float32)


def _case(w, B, pieces, cap, P, n_splits=0, out_bf16=False):
    T = sum(n for _, n in pieces)
    say("policy", w.name, f"P={P} B={B} T={T} d={w.head_dim} r={w.rank} g={w.gqa} v={w.value_dtype}",
        f"splits={n_splits}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0] if w.rank else None
    a = _direction(w)
    dc, K, V = gpu_cache(w, U, B, T, cap, pieces=pieces, value_protect=P, a_dir=a)
    oc = orc.empty_cache(B, w.n_kv_heads, cap, w.head_dim, w.rank, 1, VDT[w.value_dtype],
                         key_dtype=VDT[w.key_dtype], value_protect=P)
    for b in range(B):
        for h in range(w.n_kv_heads):
            for st, n in pieces:
                orc.write_stream(oc, b, h, st, K[b, h, st:st + n], value_payload(V[b, h, st:st + n], w),
                                 None if U is None else U[h], 1, VDT[w.value_dtype], a_h=a[h])
    compare_cache(dc, oc)
    assert np.any(oc["vpidx"] != 0)  # the choice is not trivially slot order
    q = synth.decode_queries(w, position=T, batch=B)
    lg, out = decode_gpu(dc, w, q, T, out_bf16=out_bf16, n_splits=n_splits)
    ref_l, ref_o = orc.decode(oc, q, U, T, 1.0, 1, VDT[w.value_dtype])
    check_logits(lg, ref_l)
    check_out(out, ref_o, out_bf16)
    # the corrections matter: the oracle's decode without them differs by more than the tolerance
    if P:
        plain = {k: v for k, v in oc.items() if k not in ("vpidx", "vprot")}
        _, ref0 = orc.decode(plain, q, U, T, 1.0, 1, VDT[w.value_dtype])
        assert np.max(np.abs(ref0 - ref_o)) > 0


@pytest.mark.parametrize("P", [1, 2])
def test_fullkv_shape_two_groups_share_columns(P):
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2)
    _case(w, 2, [(0, 96), (96, 37)], 160, P)


@pytest.mark.parametrize("P", [1, 2])
def test_gqa16_one_group_per_product_f32_values_splits(P):
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=32, n_kv_heads=2, value_dtype="f32", key_dtype="f32")
    _case(w, 1, [(0, 320)], 320, P, n_splits=3, out_bf16=True)


@pytest.mark.parametrize("P", [1, 2])
def test_d64_gqa8(P):
    w = synth.scaled(W["tinyllama_decode"], value_mode="q2", n_q_heads=16, n_kv_heads=2)
    _case(w, 2, [(0, 64), (64, 1), (65, 200)], 288, P, n_splits=2)


def test_gqa7_long_context_rank32():
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=14, n_kv_heads=2, rank=32)
    _case(w, 1, [(0, 1000)], 1024, 2)


def test_long_write_two_groups_per_workgroup():
    """More than 2048 groups in one append (the long-write workgroup shape)."""
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=20, n_kv_heads=4)
    _case(w, 2, [(0, 8256)], 8256, 2)


def test_paged_ragged_rows():
    from .test_gpu_paged import _run
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2)
    _run(w, 3, 160, (40, 1, 30, 33, 2), out_bf16=True, value_protect=2, a_dir=_direction(w))


@pytest.mark.parametrize("P", [1, 2])
def test_chunked_prefill_with_corrections(P):
    """The chunked prefill reads the corrections as the decode does: logits and outputs of sampled
    query tokens against the oracle's prefill over its own policy cache."""
    import torch
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2)
    B, start, n_q, cap = 2, 70, 40, 128
    L = start + n_q
    say("policy-prefill", w.name, f"P={P} B={B} start={start} n_q={n_q}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0]
    a = _direction(w)
    pieces = [(0, 64), (64, 6), (70, 40)]
    dc, K, V = gpu_cache(w, U, B, L, cap, pieces=pieces, value_protect=P, a_dir=a)
    oc = orc.empty_cache(B, w.n_kv_heads, cap, w.head_dim, w.rank, 1, VDT[w.value_dtype],
                         key_dtype=VDT[w.key_dtype], value_protect=P)
    for b in range(B):
        for h in range(w.n_kv_heads):
            for st, n in pieces:
                orc.write_stream(oc, b, h, st, K[b, h, st:st + n], value_payload(V[b, h, st:st + n], w), U[h], 1,
                                 VDT[w.value_dtype], a_h=a[h])
    compare_cache(dc, oc)
    q = synth.decode_queries(w, batch=B * n_q, stream=5).reshape(B, n_q, w.n_q_heads, w.head_dim)
    lg = torch.full((B, n_q, w.n_q_heads, L), float("nan"), device="cuda")
    out = dc.prefill(to_device(q, w.query_dtype), start, logits_dbg=lg)
    torch.cuda.synchronize()
    lg, out = lg.cpu().numpy(), out.float().cpu().numpy()
    tokens = [0, 7, 25, 39]
    ref_l, ref_o = orc.prefill(oc, q, U, start, 1.0, 1, VDT[w.value_dtype], tokens=tokens)
    for t in tokens:
        check_logits(lg[:, t, :, :start + t + 1], ref_l[:, t, :, :start + t + 1])
        check_out(out[:, t], ref_o[:, t], False)


@pytest.mark.parametrize("P", [0, 2])
def test_diagnostics_a2_with_corrections(P):
    """The score-space diagnostics read the corrections: every statistic against the oracle's
    (whose value rows carry them), and A^2 falls when the policy is on."""
    from .test_gpu_diagnostics import check_stats
    from oracle import diagnostics as dg
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2)
    B, T = 2, 200
    say("policy-diagnostics", w.name, f"P={P} B={B} T={T}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0]
    a = _direction(w)
    pieces = [(0, 192), (192, 8)]
    dc, K, V = gpu_cache(w, U, B, T, 224, pieces=pieces, value_protect=P, a_dir=a)
    oc = orc.empty_cache(B, w.n_kv_heads, 224, w.head_dim, w.rank, 1, VDT[w.value_dtype],
                         key_dtype=VDT[w.key_dtype], value_protect=P)
    for b in range(B):
        for h in range(w.n_kv_heads):
            for st, n in pieces:
                orc.write_stream(oc, b, h, st, K[b, h, st:st + n], value_payload(V[b, h, st:st + n], w), U[h], 1,
                                 VDT[w.value_dtype], a_h=a[h])
    q = synth.decode_queries(w, position=T, batch=B)
    got = dc.score_diagnostics(to_device(q, w.query_dtype), to_device(K, w.key_dtype), to_device(V, w.value_dtype),
                               T).cpu().numpy()
    ref = dg.score_diagnostics(oc, q, U, T, 1.0, K, V, 1, VDT[w.value_dtype])
    check_stats(got, ref)
    if P:
        plain = {k: v for k, v in oc.items() if k not in ("vpidx", "vprot")}
        ref0 = dg.score_diagnostics(plain, q, U, T, 1.0, K, V, 1, VDT[w.value_dtype])
        assert np.mean(ref[..., 4]) < np.mean(ref0[..., 4])
