"""GPU parity of the 3- and 4-bit base-code variants (one code per nibble).

The base quantizer at 3 and 4 bits (7 and 15 levels) through every kernel that reads or writes key
codes: the append (both workgroup shapes) bit-exact against the oracle, the matrix-core decode
(dense bf16 and 2-bit values), the vector decode (f32 values), paged caches, the chunked prefill
and the score-space diagnostics, each to the tolerance of its 2-bit counterpart.
"""
import numpy as np
import pytest

from oracle import diagnostics as dg
from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import check_logits, check_out, compare_cache, decode_gpu, gpu_cache, say, to_device
from .helpers import VDT, VMODE, value_payload

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _oracle(w, U, K, V, cap, pieces):
    B, H = K.shape[:2]
    oc = orc.empty_cache(B, H, cap, w.head_dim, 0 if U is None else U.shape[2], VMODE[w.value_mode],
                         VDT[w.value_dtype], key_dtype=VDT[w.key_dtype], base_bits=w.base_bits)
    for b in range(B):
        for h in range(H):
            for st, n in pieces:
                orc.write_stream(oc, b, h, st, K[b, h, st:st + n], value_payload(V[b, h, st:st + n], w),
                                 None if U is None else U[h], VMODE[w.value_mode], VDT[w.value_dtype],
                                 bits=w.base_bits)
    return oc


def _decode_case(w, B, pieces, cap, out_bf16=False, n_splits=0):
    T = sum(n for _, n in pieces)
    say("decode", w.name, f"bits={w.base_bits} B={B} T={T} d={w.head_dim} r={w.rank} g={w.gqa}",
        f"v={w.value_mode}/{w.value_dtype} splits={n_splits}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0] if w.rank else None
    dc, K, V = gpu_cache(w, U, B, T, cap, pieces=pieces)
    oc = _oracle(w, U, K, V, cap, pieces)
    compare_cache(dc, oc)
    q = synth.decode_queries(w, position=T, batch=B)
    lg, out = decode_gpu(dc, w, q, T, out_bf16=out_bf16, n_splits=n_splits)
    ref_l, ref_o = orc.decode(oc, q, U, T, 1.0, VMODE[w.value_mode], VDT[w.value_dtype])
    check_logits(lg, ref_l)
    check_out(out, ref_o, out_bf16)


@pytest.mark.parametrize("bits", [3, 4])
def test_qwen7b_shape_matrix_core_decode(bits):
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2, base_bits=bits)
    _decode_case(w, 2, [(0, 96), (96, 37)], 160)


@pytest.mark.parametrize("bits", [3, 4])
def test_fullkv_two_bit_values(bits):
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2, base_bits=bits)
    _decode_case(w, 2, [(0, 128), (128, 5)], 160, out_bf16=True)


@pytest.mark.parametrize("bits", [3, 4])
def test_tinyllama_shape_d64(bits):
    w = synth.scaled(W["tinyllama_decode"], n_q_heads=16, n_kv_heads=2, base_bits=bits)
    _decode_case(w, 2, [(0, 64), (64, 31)], 96)


@pytest.mark.parametrize("bits", [3, 4])
def test_tiny_f32_vector_decode(bits):
    _decode_case(synth.scaled(W["tiny"], base_bits=bits), 2, [(0, 200)], 256)


@pytest.mark.parametrize("bits", [3, 4])
def test_long_write_two_groups_per_workgroup(bits):
    """More than 2048 groups in one append: the two-groups-per-workgroup path."""
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=8, n_kv_heads=4, base_bits=bits)
    _decode_case(w, 2, [(0, 8256)], 8256)


@pytest.mark.parametrize("bits", [3, 4])
def test_prefill(bits):
    import torch
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2, base_bits=bits)
    B, start, n_q, cap = 2, 70, 40, 128
    L = start + n_q
    say("bits-prefill", w.name, f"bits={bits} B={B} start={start} n_q={n_q}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0]
    pieces = [(0, 64), (64, 6), (70, 40)]
    dc, K, V = gpu_cache(w, U, B, L, cap, pieces=pieces)
    oc = _oracle(w, U, K, V, cap, pieces)
    q = synth.decode_queries(w, batch=B * n_q, stream=5).reshape(B, n_q, w.n_q_heads, w.head_dim)
    lg = torch.full((B, n_q, w.n_q_heads, L), float("nan"), device="cuda")
    out = dc.prefill(to_device(q, w.query_dtype), start, logits_dbg=lg)
    torch.cuda.synchronize()
    lg, out = lg.cpu().numpy(), out.float().cpu().numpy()
    tokens = [0, 5, 20, 39]
    ref_l, ref_o = orc.prefill(oc, q, U, start, 1.0, 0, 1, tokens=tokens)
    for t in tokens:
        check_logits(lg[:, t, :, :start + t + 1], ref_l[:, t, :, :start + t + 1])
        check_out(out[:, t], ref_o[:, t], False)


@pytest.mark.parametrize("bits", [3, 4])
def test_score_diagnostics(bits):
    from .test_gpu_diagnostics import check_stats
    from .test_oracle_diagnostics import _build
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2, base_bits=bits)
    n_ctx = 200
    say("bits-diagnostics", w.name, f"bits={bits} n_ctx={n_ctx}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0]
    dc, K, V = gpu_cache(w, U, 2, n_ctx, 224, pieces=[(0, 192), (192, 8)])
    q = synth.decode_queries(w, position=n_ctx, batch=2)
    got = dc.score_diagnostics(to_device(q, w.query_dtype), to_device(K, w.key_dtype), to_device(V, w.value_dtype),
                               n_ctx).cpu().numpy()
    ref = dg.score_diagnostics(_build(w, U, K, V, n_ctx), q, U, n_ctx, 1.0, K, V, 0, 1)
    check_stats(got, ref)


@pytest.mark.parametrize("bits", [3, 4])
def test_paged_ragged_rows(bits):
    from .test_gpu_paged import _run
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2, base_bits=bits), 3, 128, [1, 37, 40])
