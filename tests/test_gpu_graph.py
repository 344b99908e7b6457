"""A decode step (append of the newest tokens + decode) captured in a HIP graph and replayed.

The library's calls are plain kernel launches on the caller's stream, with every buffer passed
in (no allocation, copy or memset inside), so a serving loop can capture them. Each replay must
give exactly the eager step's output (the same kernels on the same inputs), with eager library
work and host synchronizations between the replays; the eager output itself is checked against
the oracle's fp64 decode, and after the replays the cache bytes still equal the oracle's.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import check_out, compare_cache, gpu_cache, oracle_pieces, say, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.mark.parametrize("wname,B,T,new,n_splits,bf16", [
    ("qwen7b_decode", 2, 1024, 32, 3, True),       # whole groups, splits merged in-kernel
    ("qwen7b_decode", 2, 1000, 40, 0, False),      # the step also writes the unfinished group's tails
    ("qwen14b_fullkv", 1, 512, 32, 2, True),       # 2-bit values
])
def test_captured_step_replays_equal_eager(wname, B, T, new, n_splits, bf16):
    import torch
    import quantized_kv_cache_headq_amd as hq
    w = synth.scaled(W[wname])
    say("graph", wname, f"B={B} T={T} new={new} splits={n_splits} bf16out={bf16}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=256), w.n_kv_heads, w.rank)[0]
    cap = (T + 31) // 32 * 32
    start = T - new
    pieces = [(0, start), (start, new)]
    dc, K, V = gpu_cache(w, U, B, T, cap, pieces=pieces)
    Kd, Vd = to_device(K, w.key_dtype), to_device(V, w.value_dtype)
    kn, vn = Kd[:, :, start:], Vd[:, :, start:]
    q = synth.decode_queries(w, position=T, batch=B)
    qd = to_device(q, w.query_dtype)
    q2 = to_device(synth.decode_queries(w, position=T - 1, batch=B), w.query_dtype)
    odt = hq.HEADQ_BF16 if bf16 else hq.HEADQ_F32
    tdt = torch.bfloat16 if bf16 else torch.float32
    ws = torch.zeros((hq.decode_workspace_bytes(dc.cfg, T, n_splits) + 3) // 4, dtype=torch.float32, device="cuda")
    out_e = torch.empty((B, w.n_q_heads, w.head_dim), dtype=tdt, device="cuda")
    out_g = torch.empty_like(out_e)
    out_x = torch.empty_like(out_e)

    def step(s, out):
        dc.append(kn, vn, start, stream=s)
        dc.decode(qd, T, out=out, out_dtype=odt, n_splits=n_splits, ws=ws, stream=s)

    step(torch.cuda.current_stream(), out_e)
    torch.cuda.synchronize()
    oc = oracle_pieces(w, U, K, V, cap, pieces)
    _, ref = orc.decode(oc, q, U, T, 1.0, 0 if w.value_mode == "dense" else 1, 0 if w.value_dtype == "f32" else 1)
    check_out(out_e.float().cpu().numpy(), ref, bf16)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream(), out_g)
    torch.cuda.synchronize()
    eager = out_e.float().cpu().numpy()
    for rep in range(3):
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out_g.float().cpu().numpy()
        assert np.array_equal(got, eager), f"replay {rep}: max |diff| {np.nanmax(np.abs(got - eager))}"
        # eager library work between replays, on the same workspace
        dc.decode(q2, T, out=out_x, out_dtype=odt, n_splits=n_splits, ws=ws)
        torch.cuda.synchronize()
    compare_cache(dc, oc)
    assert not torch.any(ws[:B * w.n_kv_heads].view(torch.int32) != 0), "split counters not back to zero"
