"""GPU parity on the method's degenerate cases and at the split-count limit, through the C ABI.

Channels constant over their 32-token group (zero step: every code 0, the key the binary16 zero
alone), whole groups of zero keys (no residual, no side code), constant and zero value groups of
the 2-bit value quantizer, a zero query (uniform attention), keys hundreds of times larger than
the workloads' (the decode's per-head query scaling must keep q o s inside binary16), and the
largest split count the matrix-core decode takes (128, one work unit per split, the last one the
unfinished group alone). Cache bytes bit-exact, logits and outputs to the decode tolerances.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import (check_logits, check_out, compare_cache, decode_gpu, gpu_cache, oracle_pieces, say)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
G = 32


def _round_to(x, dtype_name):
    """Round f32 inputs to the stored dtype (bf16: nearest even), as the generator does."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return (t.bfloat16().float() if dtype_name == "bf16" else t).numpy()


def _degenerate(w, B, T):
    K = synth.stack_streams(w, "keys", B, T).copy()
    V = synth.stack_streams(w, "values", B, T).copy()
    d = w.head_dim
    K[:, :, :G, 3] = 1.25                  # constant over group 0
    K[:, :, :G, d // 2] = -7.3
    K[:, :, :, d - 5] = 0.1                # constant in every group
    K[:, :, :, 1] = 0.0
    K[:, :, G:2 * G] = 0.0                 # a whole group of zero keys
    V[:, :, 5, 0:32] = 0.75                # constant 32-channel value groups
    V[:, :, 9, d - 32:] = -3.0
    V[:, :, 20] = 0.0                      # a zero value row
    return _round_to(K, w.key_dtype), _round_to(V, w.value_dtype)


def _run(w, K, V, pieces, cap, queries, n_splits=0, out_bf16=False):
    T = sum(n for _, n in pieces)
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0]
    dc, _, _ = gpu_cache(w, U, K.shape[0], T, cap, K=K, V=V, pieces=pieces)
    oc = oracle_pieces(w, U, K, V, cap, pieces)
    compare_cache(dc, oc)
    for name, q in queries:
        say("edge", w.name, name, f"T={T} splits={n_splits}")
        lg, out = decode_gpu(dc, w, q, T, out_bf16=out_bf16, n_splits=n_splits)
        ref_l, ref_o = orc.decode(oc, q, U, T, 1.0, 0 if w.value_mode == "dense" else 1,
                                  0 if w.value_dtype == "f32" else 1)
        check_logits(lg, ref_l)
        check_out(out, ref_o, out_bf16)
        if name == "zero query":
            assert np.all(lg == 0.0)


@pytest.mark.parametrize("wname,kw", [
    ("qwen7b_decode", {}),
    ("qwen14b_fullkv", {}),
    ("tinyllama_decode", dict(n_q_heads=16, n_kv_heads=2)),
])
def test_degenerate_groups_and_zero_query(wname, kw):
    w = synth.scaled(W[wname], **kw)
    B, T = 2, 3 * G + 7
    K, V = _degenerate(w, B, T)
    q = synth.decode_queries(w, position=T, batch=B)
    _run(w, K, V, [(0, 3 * G), (3 * G, 7)], 4 * G,
         [("random query", q), ("zero query", np.zeros_like(q))], out_bf16=(wname != "qwen7b_decode"))


@pytest.mark.parametrize("wname", ["qwen7b_decode", "qwen14b_fullkv"])
def test_large_magnitude_keys(wname):
    w = synth.scaled(W[wname])
    B, T = 1, 4 * G + 3
    K = _round_to(300.0 * synth.stack_streams(w, "keys", B, T), w.key_dtype)
    V = synth.stack_streams(w, "values", B, T)
    assert np.abs(K).max() < 65504.0 / 2  # the channel ranges stay inside binary16
    q = synth.decode_queries(w, position=T, batch=B)
    _run(w, K, V, [(0, 4 * G), (4 * G, 3)], 5 * G, [("random query", q)])


@pytest.mark.parametrize("wname", ["qwen7b_decode", "qwen14b_fullkv"])
def test_split_count_limit(wname):
    w = synth.scaled(W[wname], n_q_heads=W[wname].gqa, n_kv_heads=1)
    B, T = 1, 127 * G + 5                  # 128 work units: 127 whole groups and the tail
    K = synth.stack_streams(w, "keys", B, T)
    V = synth.stack_streams(w, "values", B, T)
    q = synth.decode_queries(w, position=T, batch=B)
    _run(w, K, V, [(0, 127 * G), (127 * G, 5)], 128 * G, [("random query", q)], n_splits=128, out_bf16=True)
