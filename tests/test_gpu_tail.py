"""GPU parity of token-granular cache writes and of decoding an unfinished last group.

Appends of any length (one token at a time, runs that finish groups and start new ones) must
leave every cache buffer, the dense tails included, bit-exact with the oracle fed the same pieces;
decodes at lengths that end inside a group read those tokens exactly from the tails and must match
the oracle's logits and outputs within the same tolerances as whole groups.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import check_logits, check_out, compare_cache, decode_gpu, gpu_cache, say
from .helpers import VDT, VMODE, value_payload

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _oracle_pieces(w, U, K, V, cap, pieces):
    B, H = K.shape[:2]
    oc = orc.empty_cache(B, H, cap, w.head_dim, 0 if U is None else U.shape[2], VMODE[w.value_mode],
                         VDT[w.value_dtype], key_dtype=VDT[w.key_dtype])
    for b in range(B):
        for h in range(H):
            for start, n in pieces:
                orc.write_stream(oc, b, h, start, K[b, h, start:start + n],
                                 value_payload(V[b, h, start:start + n], w), None if U is None else U[h],
                                 VMODE[w.value_mode], VDT[w.value_dtype])
    return oc


def _run(w, B, cap, pieces, decode_at, out_bf16=False, n_splits=0):
    say("tail", w.name, f"B={B} cap={cap} d={w.head_dim} r={w.rank} g={w.gqa} v={w.value_mode}/{w.value_dtype}",
        f"pieces={pieces} decode_at={decode_at} splits={n_splits}")
    T = sum(n for _, n in pieces)
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0] if w.rank else None
    done = []
    dc = K = V = None
    for i in range(len(pieces)):
        # grow the cache piece by piece on both sides, checking after each piece
        if dc is None:
            dc, K, V = gpu_cache(w, U, B, T, cap, pieces=pieces[:1])
        else:
            import quantized_kv_cache_headq_amd as hq  # noqa: F401
            from .gpu_helpers import to_device
            start, n = pieces[i]
            dc.append(to_device(K[:, :, start:start + n], w.key_dtype), to_device(V[:, :, start:start + n],
                                                                                 w.value_dtype), start)
        done.append(pieces[i])
        n_ctx = sum(n for _, n in done)
        oc = _oracle_pieces(w, U, K, V, cap, done)
        compare_cache(dc, oc)
        if n_ctx in decode_at:
            q = synth.decode_queries(w, position=n_ctx, batch=B)
            lg, out = decode_gpu(dc, w, q, n_ctx, out_bf16=out_bf16, n_splits=n_splits)
            ref_l, ref_o = orc.decode(oc, q, U, n_ctx, 1.0, VMODE[w.value_mode], VDT[w.value_dtype])
            check_logits(lg, ref_l)
            check_out(out, ref_o, out_bf16)


PIECES = [(0, 40), (40, 1), (41, 19), (60, 36), (96, 5), (101, 1)]


def test_qwen7b_shape_token_granular():
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2)
    _run(w, 2, 128, PIECES, {40, 41, 60, 96, 101, 102})


def test_fullkv_two_bit_token_granular():
    w = synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2)
    _run(w, 2, 128, PIECES, {41, 96, 102}, out_bf16=True)


def test_tinyllama_shape_token_granular_d64():
    w = synth.scaled(W["tinyllama_decode"], n_q_heads=16, n_kv_heads=2)
    _run(w, 2, 128, PIECES, {41, 102})


def test_tiny_f32_token_granular_vector_kernel():
    _run(W["tiny"], 1, 128, [(0, 5), (5, 27), (32, 33), (65, 3)], {5, 32, 65, 68})


def test_context_inside_the_tail_only():
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1)
    _run(w, 1, 64, [(0, 1), (1, 12), (13, 18)], {1, 13, 31})


@pytest.mark.parametrize("splits", [1, 3])
def test_tail_with_splits(splits):
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2, rank=32)
    _run(w, 1, 640, [(0, 512), (512, 17)], {529}, n_splits=splits)


def test_ragged_rows_per_row_positions_and_lengths():
    """Rows at different lengths: appends at per-row positions (device row_start), decode of
    per-row lengths (device row_len), against the oracle fed row by row."""
    import torch
    import quantized_kv_cache_headq_amd as hq
    from .gpu_helpers import config, to_device
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2)
    B, cap = 3, 192
    say("ragged", w.name, f"B={B} cap={cap}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0]
    Kf = synth.stack_streams(w, "keys", B, cap)
    Vf = synth.stack_streams(w, "values", B, cap)
    dc = hq.DeviceCache(config(w, B, cap))
    dc.set_basis(U)
    oc = orc.empty_cache(B, w.n_kv_heads, cap, w.head_dim, w.rank, VMODE[w.value_mode], VDT[w.value_dtype],
                         key_dtype=VDT[w.key_dtype])
    lengths = np.array([0, 3, 7])  # rows 1 and 2 start inside group 0 (earlier rows read as zeros)
    for n_new in (33, 1, 1, 40, 24, 1):
        K = np.stack([Kf[b, :, lengths[b]:lengths[b] + n_new] for b in range(B)])
        V = np.stack([Vf[b, :, lengths[b]:lengths[b] + n_new] for b in range(B)])
        rs = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        dc.append(to_device(K, w.key_dtype), to_device(V, w.value_dtype), 0, row_start=rs)
        for b in range(B):
            for h in range(w.n_kv_heads):
                orc.write_stream(oc, b, h, int(lengths[b]), K[b, h], value_payload(V[b, h], w), U[h],
                                 VMODE[w.value_mode], VDT[w.value_dtype])
        lengths = lengths + n_new
        compare_cache(dc, oc)
        n_max = int(lengths.max())
        q = synth.decode_queries(w, position=n_max, batch=B)
        rl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        qd = to_device(q, w.query_dtype)
        lg = torch.full((B, w.n_q_heads, n_max), float("nan"), device="cuda")
        out = dc.decode(qd, n_max, logits_dbg=lg, row_len=rl)
        torch.cuda.synchronize()
        ref_l, ref_o = orc.decode(oc, q, U, n_max, 1.0, VMODE[w.value_mode], VDT[w.value_dtype], row_len=lengths)
        lg = lg.cpu().numpy()
        for b in range(B):
            check_logits(lg[b, :, :lengths[b]], ref_l[b, :, :lengths[b]])
        check_out(out.float().cpu().numpy(), ref_o, False)
