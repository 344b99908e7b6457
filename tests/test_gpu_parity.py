"""GPU parity of libheadq against the CPU oracle, through the C ABI.

Packed cache bytes must be bit-exact; decode logits within 1e-3 * max(1, |s|) (natural-log
units) and outputs within 2e-3 absolute (plus half a bf16 ulp for bf16 output), against the
oracle's fp64 decode of its own independently packed cache built from the same seeded inputs.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import (check_logits, check_out, compare_cache, decode_gpu, gpu_cache, oracle_for, say)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _case(w, B, T, cap=None, n_ctx=None, corr=1.0, out_bf16=False, n_splits=0, pieces=None):
    cap = T if cap is None else cap
    n_ctx = T if n_ctx is None else n_ctx
    say(w.name, f"B={B} T={T} cap={cap} n_ctx={n_ctx} r={w.rank} d={w.head_dim} g={w.gqa} v={w.value_mode}",
        f"corr={corr} bf16out={out_bf16} splits={n_splits}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=256), w.n_kv_heads, w.rank)[0] if w.rank else None
    dc, K, V = gpu_cache(w, U, B, T, cap, pieces=pieces)
    oc = oracle_for(w, U, K, V, cap)
    compare_cache(dc, oc)
    q = synth.decode_queries(w, position=n_ctx, batch=B)
    lg, out = decode_gpu(dc, w, q, n_ctx, out_bf16=out_bf16, corr=corr, n_splits=n_splits)
    ref_l, ref_o = orc.decode(oc, q, U, n_ctx, corr, 0 if w.value_mode == "dense" else 1,
                              0 if w.value_dtype == "f32" else 1)
    check_logits(lg, ref_l)
    check_out(out, ref_o, out_bf16)
    return dc, q, out


def test_tiny_fp32():
    _case(W["tiny"], 1, 256)


def test_tinyllama_shape_small():
    _case(synth.scaled(W["tinyllama_decode"], batch=2), 2, 512, cap=640, n_ctx=480)


def test_qwen7b_shape_small():
    _case(synth.scaled(W["qwen7b_decode"]), 2, 1024)


def test_qwen7b_shape_bf16_out_ragged_splits():
    _case(synth.scaled(W["qwen7b_decode"]), 1, 704, cap=1024, out_bf16=True, n_splits=5)


def test_append_prefill_shape_small():
    _case(synth.scaled(W["append_prefill"]), 1, 2048)


def test_fullkv_two_bit_values_small():
    _case(synth.scaled(W["qwen14b_fullkv"]), 1, 512)


def test_fullkv_two_bit_values_d64_ragged_splits():
    w = synth.scaled(W["tinyllama_decode"], value_mode="q2", batch=2)
    _case(w, 2, 512, cap=640, n_ctx=416, out_bf16=True, n_splits=3)


@pytest.mark.parametrize("rank", [0, 32])
def test_fullkv_two_bit_values_ranks(rank):
    _case(synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2, rank=rank), 1, 384, n_splits=2)


def test_fullkv_two_bit_values_f32_input_gqa16():
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=32, n_kv_heads=2, value_dtype="f32", key_dtype="f32")
    _case(w, 1, 256)


@pytest.mark.parametrize("rank", [0, 4, 8, 32])
def test_rank_variants(rank):
    _case(synth.scaled(W["qwen7b_decode"], n_q_heads=8, n_kv_heads=2, rank=rank), 1, 256)


@pytest.mark.parametrize("corr", [0.0, -1.0, 0.5, 2.5])
def test_correction_scale_controls(corr):
    _case(synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2), 1, 256, corr=corr)


@pytest.mark.parametrize("corr", [0.0, 0.5])
def test_correction_scale_packed_columns(corr):
    """The 2-bit value decode with three groups sharing the matrix columns, at other scales."""
    _case(synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2), 1, 384 + 32, corr=corr, n_splits=2)


def test_append_in_pieces_at_offsets():
    w = synth.scaled(W["tinyllama_decode"], n_q_heads=8, n_kv_heads=2)
    _case(w, 2, 384, cap=448, pieces=[(0, 128), (128, 32), (160, 224)])


def test_d64_gqa16():
    _case(synth.scaled(W["tinyllama_decode"], n_q_heads=32, n_kv_heads=2), 1, 256)


def test_strided_keys_and_values():
    """Keys/values passed as non-contiguous views (token stride larger than d)."""
    import torch
    import quantized_kv_cache_headq_amd as hq
    from .gpu_helpers import config, to_device
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1)
    say("strided", w.name)
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), 1, w.rank)[0]
    K = synth.stack_streams(w, "keys", 2, 128)
    V = synth.stack_streams(w, "values", 2, 128)
    big = torch.zeros((2, 1, 128, 3 * 128), dtype=torch.bfloat16, device="cuda")
    big[..., 128:256] = to_device(K, "bf16")
    bigv = torch.zeros((2, 1, 128, 2 * 128), dtype=torch.bfloat16, device="cuda")
    bigv[..., 128:] = to_device(V, "bf16")
    dc = hq.DeviceCache(config(w, 2, 128))
    dc.set_basis(U)
    dc.append(big[..., 128:256], bigv[..., 128:], 0)
    compare_cache(dc, oracle_for(w, U, K, V, 128))


def test_split_count_invariance_and_determinism():
    """Splitting the tokens differently only changes rounding. The matrix-core path carries each
    probability as bf16 hi + lo (relative representation error <= 2^-18), so two split counts may
    differ by up to 2 * max|v| * 2^-18 (plus f32 accumulation rounding); the same split count is
    bit-stable."""
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2)
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), 2, w.rank)[0]
    say("splits", w.name)
    dc, K, V = gpu_cache(w, U, 1, 2048)
    q = synth.decode_queries(w, batch=1)
    _, ref = decode_gpu(dc, w, q, 2048, n_splits=1, logits=False)
    for s in (2, 7, 16, 64):
        _, o = decode_gpu(dc, w, q, 2048, n_splits=s, logits=False)
        bound = 2 * float(np.abs(V).max()) * 2.0 ** -18 + 2e-6
        assert np.max(np.abs(o - ref)) <= bound, (s, np.max(np.abs(o - ref)), bound)
    _, a = decode_gpu(dc, w, q, 2048, logits=False)
    for _ in range(3):
        _, b = decode_gpu(dc, w, q, 2048, logits=False)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_workspace_counters_return_to_zero_and_reuse():
    """The split merge counts workgroups in on the workspace; every call must leave the counter
    region zero so one zeroed workspace serves calls with different split counts."""
    import torch
    import quantized_kv_cache_headq_amd as hq
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2)
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), 2, w.rank)[0]
    say("workspace reuse", w.name)
    dc, K, V = gpu_cache(w, U, 2, 1024)
    q = synth.decode_queries(w, batch=2)
    from .gpu_helpers import to_device
    qd = to_device(q, "bf16")
    nb = max(hq.decode_workspace_bytes(dc.cfg, 1024, s) for s in (1, 3, 8, 32))
    ws = torch.zeros((nb + 3) // 4, dtype=torch.float32, device="cuda")
    oc = oracle_for(w, U, K, V, 1024)
    _, ref = orc.decode(oc, q, U, 1024, 1.0, 0, 1, want_logits=False)
    for s in (1, 3, 8, 32, 0, 3):
        out = dc.decode(qd, 1024, n_splits=s, ws=ws)
        torch.cuda.synchronize()
        check_out(out.cpu().numpy(), ref, False)
        assert int(ws[:64].abs().sum().item()) == 0, f"counters not reset after n_splits={s}"


@pytest.mark.parametrize("g,d,T,splits", [(7, 128, 213, 2), (8, 64, 40, 0), (3, 128, 352, 3), (2, 128, 1000, 0),
                                          (5, 128, 45, 1), (6, 64, 300, 2), (4, 128, 96, 3)])
def test_packed_columns_two_bit_values(g, d, T, splits):
    """2-bit values with g <= 8: 16 // g groups (at most 3) share the matrix columns. Ragged ends
    (steps with fewer groups than columns blocks, waves without groups), a dense tail, padding
    columns, splits."""
    base = W["qwen14b_fullkv"] if d == 128 else synth.scaled(W["tinyllama_decode"], value_mode="q2")
    w = synth.scaled(base, n_q_heads=2 * g, n_kv_heads=2)
    from .test_gpu_bits import _decode_case
    n_full = T // 32 * 32
    pieces = [p for p in [(0, n_full), (n_full, T - n_full)] if p[1]]
    _decode_case(w, 2, pieces, (T + 31) // 32 * 32, out_bf16=g % 2 == 0, n_splits=splits)
