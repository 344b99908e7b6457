"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle cannot decode a whole full-size batch in seconds, so it re-encodes a few sampled
(b, h) streams itself from the generator (never from GPU output), and the GPU's cache bytes and
outputs for those streams are compared with it.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import check_logits, check_out, config, decode_gpu, gpu_cache, host, say, to_device
from .helpers import oracle_cache

pytestmark = pytest.mark.gpu


def _sampled(wname, streams, out_bf16=False, batch=None, n_splits=0):
    w = synth.WORKLOADS[wname] if isinstance(wname, str) else wname
    if batch is not None:
        w = synth.scaled(w, batch=batch)
    say("fullsize", w.name, f"B={w.batch} T={w.n_ctx} streams={streams} splits={n_splits or 'auto'}")
    U = orc.calibrate(synth.calibration_queries(w), w.n_kv_heads, w.rank)[0]
    dc, K, V = gpu_cache(w, U)
    q = synth.decode_queries(w)
    lg, out = decode_gpu(dc, w, q, w.n_ctx, out_bf16=out_bf16, n_splits=n_splits)
    g = w.gqa
    for b, h in streams:
        # oracle cache with a single batch row holding stream (b, h) at KV head h
        kv = {(0, hh): (K[b, hh], V[b, hh]) for hh in range(w.n_kv_heads)}
        wb = synth.scaled(w, batch=1)
        oc, _ = oracle_cache(wb, U, batch=1, kv=kv)
        for name in ("kcode", "kmeta", "scode", "ssc", "v", "vcode", "vmeta"):
            if name in oc:
                oc[name] = oc[name][:, h:h + 1]
        heads = list(range(h * g, (h + 1) * g))
        ref_l, ref_o = orc.decode(oc, q[b:b + 1, heads], U[h:h + 1], w.n_ctx, 1.0,
                                  0 if w.value_mode == "dense" else 1, 0 if w.value_dtype == "f32" else 1)
        check_logits(lg[b, heads], ref_l[0])
        check_out(out[b, heads], ref_o[0], out_bf16)
        compare_cache_stream(dc, oc, b, h)


def compare_cache_stream(dc, oc_one, b, h):
    """GPU stream (b, h) against the oracle's single-stream cache, bit for bit."""
    for name in ("kcode", "kmeta", "scode", "ssc", "v", "vcode", "vmeta"):
        t = getattr(dc, name)
        if t is None or name not in oc_one:
            continue
        g = host(t[b:b + 1, h:h + 1])
        o = oc_one[name]
        if name == "v" and g.dtype == np.float32:
            g, o = g.view(np.uint32), o.view(np.uint32)
        assert np.array_equal(g, o), name


def test_qwen7b_decode_full_size_sampled():
    _sampled("qwen7b_decode", [(0, 0), (31, 3), (17, 2)])


def test_tinyllama_decode_full_size_sampled():
    _sampled("tinyllama_decode", [(0, 0), (15, 3)], out_bf16=True)


def test_qwen14b_fullkv_full_context_sampled():
    """Full 32K context of the 2-bit full-KV workload in its benchmark launch shape (one
    workgroup of four waves per stream: 64 x 8 streams give one split each); the batch is cut to
    4 rows, which leaves every stream's work unchanged."""
    _sampled("qwen14b_fullkv", [(0, 0), (3, 7), (2, 5)], out_bf16=True, batch=4, n_splits=1)


def test_long_f32_write_two_groups_per_workgroup():
    """A write of more than 2048 groups takes the long-write append (two groups per workgroup,
    U_h through scalar loads); f32 keys and values, so also the vector decode kernel."""
    w = synth.scaled(synth.WORKLOADS["tiny"], n_q_heads=8, n_kv_heads=4, batch=8, n_ctx=4096)
    _sampled(w, [(0, 0), (7, 3), (4, 1)])


def _one_stream(oc, h):
    """KV head h of a one-row oracle cache, as a cache of its own."""
    return {k: np.ascontiguousarray(v[:, h:h + 1]) for k, v in oc.items()}


def test_append_prefill_full_size_sampled():
    """The prefill write as the benchmark times it: all 32768 tokens of all 8 KV heads (rank 32,
    bf16 keys) in one append of keys alone, two groups per workgroup; sampled heads re-encoded
    by the oracle and compared byte for byte."""
    import torch

    import quantized_kv_cache_headq_amd as hq
    w = synth.WORKLOADS["append_prefill"]
    say("fullsize", w.name, f"Hkv={w.n_kv_heads} T={w.n_ctx} r={w.rank} keys only")
    U = orc.calibrate(synth.calibration_queries(w), w.n_kv_heads, w.rank)[0]
    K = synth.stack_streams(w, "keys")
    dc = hq.DeviceCache(config(w))
    dc.set_basis(U)
    dc.append(to_device(K, w.key_dtype), None, 0)
    torch.cuda.synchronize()
    kv = {(0, hh): (K[0, hh], np.zeros_like(K[0, hh])) for hh in range(w.n_kv_heads)}
    oc, _ = oracle_cache(w, U, batch=1, kv=kv)
    for h in (0, 3, 7):
        for name in ("kcode", "kmeta", "scode", "ssc"):
            g = host(getattr(dc, name)[0:1, h:h + 1])
            assert np.array_equal(g, oc[name][:, h:h + 1]), (name, h)


def test_prefill_full_size_sampled():
    """The chunked prefill as the benchmark times it: a 512-token chunk at positions 15872..16383
    of the Qwen2.5-7B-shaped cache (batch 4, one launch, bf16 output); sampled (row, KV head,
    query token) outputs against the oracle's prefill of that stream."""
    import torch

    import quantized_kv_cache_headq_amd as hq
    B, n_q = 4, 512
    w = synth.scaled(synth.WORKLOADS["qwen7b_decode"], batch=B)
    say("fullsize prefill", w.name, f"B={B} context={w.n_ctx} chunk={n_q}")
    U = orc.calibrate(synth.calibration_queries(w), w.n_kv_heads, w.rank)[0]
    dc, K, V = gpu_cache(w, U)
    start = w.n_ctx - n_q
    qh = synth.decode_queries(w, batch=B * n_q, stream=7).reshape(B, n_q, w.n_q_heads, w.head_dim)
    out = torch.empty((B, n_q, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    hq.headq_prefill_attn(dc.cfg, dc.c(), to_device(qh, w.query_dtype), start, out, hq.HEADQ_BF16)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    g = w.gqa
    tokens = [0, 255, 511]
    for b, h in [(0, 0), (3, 2)]:
        kv = {(0, hh): (K[b, hh], V[b, hh]) for hh in range(w.n_kv_heads)}
        oc, _ = oracle_cache(synth.scaled(w, batch=1), U, batch=1, kv=kv)
        heads = list(range(h * g, (h + 1) * g))
        _, ref = orc.prefill(_one_stream(oc, h), qh[b:b + 1][:, :, heads], U[h:h + 1], start, 1.0, 0, 1,
                             tokens=tokens)
        for t in tokens:
            check_out(o[b, t, heads], ref[0, t], True)
