"""Benchmark of the HeadQ hot path on one MI355X.

python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload qwen7b_decode] [--no-cpu-baseline]

Decode workloads (qwen7b_decode, the default; tinyllama_decode; qwen14b_fullkv): one step is one
decode step through libheadq, per layer headq_cache_append of the newest 32-token group of every
(b, h) stream, then headq_decode_attn over the whole context (tinyllama_decode runs its 22 layers,
each on its own cache). append_prefill: one step is headq_cache_append of the whole prefill.
qwen7b_diagnostics: one step is headq_score_diagnostics over the full Qwen2.5-7B-shaped cache
against the keys and values it was written from (calibration-sweep diagnostics).
qwen7b_prefill: one step is headq_prefill_attn of a 512-token chunk at the end of a 16384-token
Qwen2.5-7B-shaped context (batch 4), the chunk's keys and values already appended.
The calibration (host PCA) runs once before timing, as the method prescribes (offline), and is
reported separately. Inputs are seeded synthetic tensors resident in HBM before timing starts;
several cache copies are rotated so the 256 MB MALL cannot hold the working set.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3     # 256 CU x 64 lanes x 2 (packed pair) x 2 flop per fma x 2.4 GHz
FP32_NONPACKED_PEAK_TFLOPS = 78.6   # the same without packed-fp32 instructions
METRIC = "decode-attn cached tokens·heads/s + achieved HBM GB/s (% of peak), 1 GPU"
CSRC = os.path.join(ROOT, "quantized_kv_cache_headq_amd", "csrc")
# committed rocprofv3 counter summaries per workload: (file, source of the kernel they measured)
TRAFFIC = {
    "qwen7b_decode": ("decode_qwen7b_traffic.json", "decode_mfma.hip"),
    "qwen14b_fullkv": ("decode_qwen14b_fullkv_traffic.json", "decode_mfma.hip"),
    "tinyllama_decode": ("decode_tinyllama_traffic.json", "decode_mfma.hip"),
    "append_prefill": ("append_prefill_traffic.json", "append.hip"),
    "qwen7b_diagnostics": ("diagnostics_qwen7b_traffic.json", "diagnostics.hip"),
    "qwen14b_fullkv_diagnostics": ("diagnostics_qwen14b_fullkv_traffic.json", "diagnostics.hip"),
    "qwen7b_prefill": ("prefill_qwen7b_traffic.json", "prefill_mfma.hip"),
}


def algorithmic_bytes_per_token_head(w, value_protect: int = 0) -> float:
    """Bytes the method must move per cached token per KV head (keys, side code, values; with the
    A^2 value policy also each group's P bfloat16 correction rows and its index word)."""
    d, r = w.head_dim, w.rank
    k = d // 4 + d // 8 + r // 2 + (2 if r else 0)  # 2-bit codes, fp16 step/zero per 32 tokens, nibbles, sigma
    if w.value_mode == "dense":
        v = d * (4 if w.value_dtype == "f32" else 2)
    else:
        v = d // 4 + d // 8  # 2-bit codes, fp16 step/zero per 32 channels
    if value_protect:
        return k + v + (value_protect * d * 2 + 4) / 32
    return k + v


def append_bytes(w) -> int:
    """Bytes per token per KV head of a key append: keys in, codes, step/zero, nibbles, sigma out."""
    d, r = w.head_dim, w.rank
    kin = d * (4 if w.key_dtype == "f32" else 2)
    return kin + d // 4 + d // 8 + r // 2 + (2 if r else 0)


def copy_ceiling(torch, dev, stream) -> float:
    """Read+write GB/s of a 1 GiB device-to-device copy (torch's copy kernel) on the same stream."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = 10 * 2 * src.numel() * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    return gbs


def copy_probe(torch, dev):
    """One 1 GiB device copy: the known-size reference that scales the HBM counters."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def source_sha(src: str) -> str:
    """Hash of a kernel's source file and of the library's own headers it includes."""
    h = hashlib.sha256()
    text = open(os.path.join(CSRC, src), "rb").read()
    h.update(text)
    for inc in re.findall(rb'^#include "([^"]+)"', text, flags=re.M):
        path = os.path.join(CSRC, inc.decode())
        if os.path.exists(path):
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def traffic_per_launch(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from the committed rocprofv3 counter
    summary, or None when there is none or the kernel's source changed since it was taken."""
    if workload not in TRAFFIC:
        return None
    fname, src = TRAFFIC[workload]
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", fname)))
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != source_sha(src):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, U, threads: int, rows: int, cpu_seconds: float = 15.0, value_protect: int = 0, a_dir=None):
    """The CPU oracle (as it stands) on a bounded sample: `rows` batch rows, all heads, full context,
    repeated for about `cpu_seconds` of CPU time."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import oracle as orc
    from workloads import synth

    q = synth.decode_queries(w)
    vdt = 0 if w.value_dtype == "f32" else 1
    vmode = 0 if w.value_mode == "dense" else 1
    def build(b):
        oc = orc.empty_cache(1, w.n_kv_heads, w.n_ctx, w.head_dim, w.rank, vmode, vdt, value_protect=value_protect)
        for h in range(w.n_kv_heads):
            k = synth.keys(w, b, h)
            v = synth.values(w, b, h)
            if vmode == 0 and vdt == 1:
                v = (v.view(np.uint32) >> 16).astype(np.uint16)
            orc.write_stream(oc, 0, h, 0, k, v, U[h], vmode, vdt, a_h=None if a_dir is None else a_dir[h])
        return oc

    with ThreadPoolExecutor(max_workers=threads) as ex:
        caches = list(ex.map(build, range(rows)))

    def one(b):
        orc.decode(caches[b], q[b:b + 1], U, w.n_ctx, 1.0, vmode, vdt, want_logits=False)

    # Repeat whole passes over the sample until about `cpu_seconds` of CPU time has been spent.
    passes, cpu, wall = 0, 0.0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while passes == 0 or (cpu < cpu_seconds and passes < 64):
            c0, t0 = time.process_time(), time.perf_counter()
            list(ex.map(one, range(rows)))
            cpu += time.process_time() - c0
            wall += time.perf_counter() - t0
            passes += 1
    n = passes * rows * w.n_q_heads * w.n_ctx
    # the same oracle on one thread: whole batch rows in turn for about 2 s
    rows1, wall1 = 0, 0.0
    while rows1 == 0 or (wall1 < 2.0 and rows1 < rows):
        t0 = time.perf_counter()
        one(rows1)
        wall1 += time.perf_counter() - t0
        rows1 += 1
    return {"value": n / wall, "unit": "query-head cached tokens/s", "cores": min(threads, rows), "kind": "oracle",
            "sample": f"fp64 oracle decode of {rows} of {w.batch} batch rows x {w.n_q_heads} query heads x "
                      f"{w.n_ctx} tokens, {passes} passes ({wall:.2f} s wall, {cpu:.1f} s CPU)",
            "value_one_thread": rows1 * w.n_q_heads * w.n_ctx / wall1,
            "sample_one_thread": f"{rows1} batch rows in turn on one thread ({wall1:.2f} s)"}


def append_cpu_baseline(w, U, threads: int, cpu_seconds: float = 15.0):
    """The CPU oracle's key encode (as it stands: base codes, residual, projection, side codes) of
    every KV head's whole prefill, repeated for about `cpu_seconds` of CPU time."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as orc
    from workloads import synth

    K = [synth.keys(w, 0, h) for h in range(w.n_kv_heads)]

    def one(h):
        orc.encode_keys(K[h], U[h])

    passes, cpu, wall = 0, 0.0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while passes == 0 or (cpu < cpu_seconds and passes < 64):
            c0, t0 = time.process_time(), time.perf_counter()
            list(ex.map(one, range(w.n_kv_heads)))
            cpu += time.process_time() - c0
            wall += time.perf_counter() - t0
            passes += 1
    n = passes * w.n_kv_heads * w.n_ctx
    return {"value": n / wall, "unit": "KV-head tokens/s", "cores": min(threads, w.n_kv_heads), "kind": "oracle",
            "sample": f"oracle key encode (f32) of all {w.n_kv_heads} KV heads x {w.n_ctx} tokens, rank {w.rank}, "
                      f"{passes} passes ({wall:.2f} s wall, {cpu:.1f} s CPU)"}


# diagnostics step over a decode workload's cache
DIAG_WORKLOADS = {"qwen7b_diagnostics": "qwen7b_decode", "qwen14b_fullkv_diagnostics": "qwen14b_fullkv"}
DESC = {"qwen7b_decode": "Qwen2.5-7B-shaped", "qwen14b_fullkv": "Qwen2.5-14B-shaped full-KV 2-bit"}


def diagnostics_bytes_per_token_head(w, value_protect: int = 0) -> float:
    """Bytes the diagnostics must read per token per KV head: reference keys and values, and the
    cache's keys (codes, step/zero, side code) and values (with the value policy's corrections)."""
    es = {"f32": 4, "bf16": 2}
    return w.head_dim * (es[w.key_dtype] + es[w.value_dtype]) + algorithmic_bytes_per_token_head(w, value_protect)


def diag_cpu_baseline(w, U, K, V, q, threads: int, streams: int, cpu_seconds: float = 15.0, value_protect: int = 0,
                      a_dir=None):
    """The oracle's score_diagnostics (as it stands) on a bounded sample of (b, h) streams."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import diagnostics as dg
    from oracle import oracle as orc
    from workloads import synth

    g = w.gqa
    pick = [(b % w.batch, b % w.n_kv_heads) for b in range(streams)]
    wb = synth.scaled(w, batch=1, n_kv_heads=1, n_q_heads=g)

    vmode = 0 if w.value_mode == "dense" else 1

    def build(bh):
        b, h = bh
        oc = orc.empty_cache(1, 1, w.n_ctx, w.head_dim, w.rank, vmode, 1, value_protect=value_protect)
        v = (np.ascontiguousarray(V[b, h]).view(np.uint32) >> 16).astype(np.uint16) if vmode == 0 else V[b, h]
        orc.write_stream(oc, 0, 0, 0, K[b, h], v, U[h], vmode, 1, a_h=None if a_dir is None else a_dir[h])
        return oc

    with ThreadPoolExecutor(max_workers=threads) as ex:
        caches = list(ex.map(build, pick))

    def one(i):
        b, h = pick[i]
        dg.score_diagnostics(caches[i], q[b:b + 1, h * g:(h + 1) * g], U[h:h + 1], wb.n_ctx, 1.0,
                             K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1], vmode, 1)

    passes, cpu, wall = 0, 0.0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while passes == 0 or (cpu < cpu_seconds and passes < 64):
            c0, t0 = time.process_time(), time.perf_counter()
            list(ex.map(one, range(len(pick))))
            cpu += time.process_time() - c0
            wall += time.perf_counter() - t0
            passes += 1
    n = passes * len(pick) * g * w.n_ctx
    return {"value": n / wall, "unit": "query-head cached tokens/s", "cores": min(threads, len(pick)), "kind": "oracle",
            "sample": f"fp64 oracle score_diagnostics of {len(pick)} (b, h) streams x {g} query heads x "
                      f"{w.n_ctx} tokens, {passes} passes ({wall:.2f} s wall, {cpu:.1f} s CPU)"}


MFMA_BF16_PEAK_TFLOPS = 2500.0      # dense bf16 / fp16 matrix peak
PREFILL_WORKLOADS = {"qwen7b_prefill": ("qwen7b_decode", 4, 512)}  # base shape, batch, chunk tokens


def run_prefill(args, hq, synth, torch, np):
    """One step = headq_prefill_attn of the chunk over the cache (events on the library's stream)."""
    base, B, n_q = PREFILL_WORKLOADS[args.workload]
    w = synth.scaled(synth.WORKLOADS[base], batch=B)
    dev = torch.device("cuda:0")
    DT = {"f32": hq.HEADQ_F32, "bf16": hq.HEADQ_BF16}
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    cfg = hq.Config(head_dim=w.head_dim, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, batch=B,
                    capacity=w.n_ctx, rank=w.rank, key_dtype=DT[w.key_dtype], value_dtype=DT[w.value_dtype],
                    value_mode=hq.HEADQ_V_DENSE if w.value_mode == "dense" else hq.HEADQ_V_Q2,
                    query_dtype=DT[w.query_dtype])
    U, _ = hq.headq_calibrate(cfg, synth.calibration_queries(w))
    K = torch.from_numpy(synth.stack_streams(w, "keys", workers=16)).to(dev).to(tdt[w.key_dtype])
    V = torch.from_numpy(synth.stack_streams(w, "values", workers=16)).to(dev).to(tdt[w.value_dtype])
    start = w.n_ctx - n_q
    qh = synth.decode_queries(w, batch=B * n_q, stream=7).reshape(B, n_q, w.n_q_heads, w.head_dim)
    q = torch.from_numpy(np.ascontiguousarray(qh)).to(dev).to(tdt[w.query_dtype])
    dc = hq.DeviceCache(cfg, device=dev)
    dc.set_basis(U)
    dc.append(K, V, 0)
    del K, V
    out = torch.empty((B, n_q, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    if args.copy_probe:
        copy_probe(torch, dev)

    def run():
        hq.headq_prefill_attn(cfg, dc.c(), q, start, out, hq.HEADQ_BF16, 1.0, None, stream)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms = float(step_ms.mean())
    # algorithmic work: q.k and p.v over every attended (query token, head, cached token)
    attended = sum(start + t + 1 for t in range(n_q))
    flops = 2 * 2 * w.head_dim * w.n_q_heads * B * attended
    achieved = flops / (ms / 1e3) / 1e12
    result = {
        "metric": "chunked-prefill attention query·cached-token pairs/s + achieved matrix TFLOP/s, 1 GPU",
        "value": w.n_q_heads * B * attended / (ms / 1e3), "unit": "query-head·cached-token pairs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16/bf16 operands (hi+lo), f32 accumulate", "data": "synthetic",
        "config": {"workload": f"{args.workload}: headq_prefill_attn of a {n_q}-token chunk at positions "
                               f"{start}..{w.n_ctx - 1} over the Qwen2.5-7B-shaped HeadQ cache, Hq {w.n_q_heads}, "
                               f"Hkv {w.n_kv_heads}, d {w.head_dim}, batch {B}, rank {w.rank}, dense bf16 values",
                   "batch": B, "n_q": n_q, "start": start, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "rank": w.rank, "step": "headq_prefill_attn (one launch)"},
        "roofline": {"bound": "mfma", "kernel": "prefill_mfma_kernel (one launch)", "achieved": achieved,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic_per_launch(args.workload), "algorithmic_flops_per_launch": flops,
                     "note": "every f32 factor is contracted as a high and a low half-precision part, so the "
                             "matrix cores execute at least twice the algorithmic flops"},
        "ms_p10_p90": [float(np.percentile(step_ms, 10)), float(np.percentile(step_ms, 90))],
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(w, U, start, n_q, qh, min(16, os.cpu_count() or 1))
    print(json.dumps(result), flush=True)


def prefill_cpu_baseline(w, U, start, n_q, qh, threads: int, cpu_seconds: float = 15.0):
    """The oracle's prefill (as it stands) on a bounded sample: one batch row, a few query tokens."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import oracle as orc
    from workloads import synth

    L = start + n_q
    wb = synth.scaled(w, batch=1)
    oc = orc.empty_cache(1, w.n_kv_heads, w.n_ctx, w.head_dim, w.rank, 0, 1)
    for h in range(w.n_kv_heads):
        k, v = synth.keys(wb, 0, h, L), synth.values(wb, 0, h, L)
        orc.write_stream(oc, 0, h, 0, k, (v.view(np.uint32) >> 16).astype(np.uint16), U[h], 0, 1)
    q1 = qh[:1]
    picks = list(range(n_q - 1, -1, -max(1, n_q // 16)))[:16]

    def one(t):
        orc.prefill(oc, q1, U, start, 1.0, 0, 1, tokens=[t])

    passes, cpu, wall = 0, 0.0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while passes == 0 or (cpu < cpu_seconds and passes < 64):
            c0, t0 = time.process_time(), time.perf_counter()
            list(ex.map(one, picks))
            cpu += time.process_time() - c0
            wall += time.perf_counter() - t0
            passes += 1
    pairs = passes * sum(start + t + 1 for t in picks) * w.n_q_heads
    return {"value": pairs / wall, "unit": "query-head·cached-token pairs/s", "cores": min(threads, len(picks)),
            "kind": "oracle",
            "sample": f"fp64 oracle prefill of {len(picks)} query tokens of batch row 0 x {w.n_q_heads} heads over "
                      f"the {L}-token cache, {passes} passes ({wall:.2f} s wall, {cpu:.1f} s CPU)"}


def run_diagnostics(args, hq, synth, torch, np):
    """One step = headq_score_diagnostics over the whole cache (events on the library's stream)."""
    w = synth.WORKLOADS[DIAG_WORKLOADS[args.workload]]
    dev = torch.device("cuda:0")
    DT = {"f32": hq.HEADQ_F32, "bf16": hq.HEADQ_BF16}
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    P = args.value_protect
    if P and w.value_mode != "q2":
        print("bench.py: --value-protect needs a workload with 2-bit values", file=sys.stderr)
        sys.exit(2)
    cfg = hq.Config(head_dim=w.head_dim, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, batch=w.batch,
                    capacity=w.n_ctx, rank=w.rank, key_dtype=DT[w.key_dtype], value_dtype=DT[w.value_dtype],
                    value_mode=hq.HEADQ_V_DENSE if w.value_mode == "dense" else hq.HEADQ_V_Q2,
                    query_dtype=DT[w.query_dtype], value_protect=P)
    qcal = synth.calibration_queries(w)
    U, _ = hq.headq_calibrate(cfg, qcal)
    Kh = synth.stack_streams(w, "keys", workers=16)
    Vh = synth.stack_streams(w, "values", workers=16)
    qh = synth.decode_queries(w)
    K = torch.from_numpy(Kh).to(dev).to(tdt[w.key_dtype])
    V = torch.from_numpy(Vh).to(dev).to(tdt[w.value_dtype])
    q = torch.from_numpy(qh).to(dev).to(tdt[w.query_dtype])
    dc = hq.DeviceCache(cfg, device=dev)
    dc.set_basis(U)
    a_dir = hq.headq_calibrate_mean(cfg, qcal) if P else None
    if P:
        dc.set_direction(a_dir)
    dc.append(K, V, 0)
    n_ctx = w.n_ctx
    nb = hq.diagnostics_workspace_bytes(cfg, n_ctx, args.splits)
    ws = torch.empty((nb + 7) // 8, dtype=torch.float64, device=dev)
    stats = torch.empty((w.batch, w.n_q_heads, len(hq.DIAG_STATS)), dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()
    copy_gbs = copy_ceiling(torch, dev, stream)
    if args.copy_probe:
        copy_probe(torch, dev)

    def run():
        hq.headq_score_diagnostics(cfg, dc.c(), q, K, V, n_ctx, stats, 1.0, args.splits, ws, stream)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms = float(step_ms.mean())
    per_tok = diagnostics_bytes_per_token_head(w, P)
    alg = per_tok * w.batch * w.n_kv_heads * n_ctx
    achieved = alg / (ms / 1e3) / 1e9
    tok_heads = w.batch * w.n_q_heads * n_ctx
    result = {
        "metric": "score-diagnostics cached tokens·heads/s + achieved HBM GB/s (% of peak), 1 GPU",
        "value": tok_heads / (ms / 1e3), "unit": "query-head cached tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"{args.workload}: headq_score_diagnostics (Fisher variance, KL, A^2, entropy) over "
                               f"the {DESC[w.name]} cache, Hq {w.n_q_heads}, Hkv {w.n_kv_heads}, d {w.head_dim}, "
                               f"batch {w.batch}, context {n_ctx}, rank {w.rank}, bf16 reference keys and values"
                               + (f", A^2 value policy ({P} corrected tokens per group)" if P else ""),
                   "batch": w.batch, "n_ctx": n_ctx, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "rank": w.rank, "n_splits": args.splits or "auto", "value_protect": P,
                   "step": "headq_score_diagnostics (query prep, value errors, stream pass, split merge)"},
        "roofline": {"bound": "hbm", "kernel": "headq_score_diagnostics (four launches, timed together)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if P else traffic_per_launch(args.workload), "algorithmic_bytes_per_launch": alg,
                     "bytes_per_token_kv_head": per_tok,
                     "copy_ceiling_gbs": copy_gbs},
        "ms_p10_p90": [float(np.percentile(step_ms, 10)), float(np.percentile(step_ms, 90))],
        "wall_s_timed": wall,
        # the statistics themselves, mean over (batch row, query head) of the last call
        "stats_mean": dict(zip(hq.DIAG_STATS, np.nanmean(stats.cpu().numpy().reshape(-1, len(hq.DIAG_STATS)),
                                                           axis=0).tolist())),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = diag_cpu_baseline(w, U, Kh, Vh, qh, min(16, os.cpu_count() or 1), 16, value_protect=P,
                                                   a_dir=a_dir)
    print(json.dumps(result), flush=True)


def time_graphs(torch, np, run, stream, n_caches, n_layers, args, tok_heads, eager_ms):
    """The step (every layer's append and decode) captured once per cache rotation in a HIP graph
    and replayed: the eager step time minus the replayed one is the host launch overhead. The
    library's calls are plain kernel launches on the given stream (no allocation, copy or memset),
    so they capture as they are."""
    period = n_caches // math.gcd(n_caches, n_layers)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(period):
            run(i, stream=side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(period):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(i, stream=torch.cuda.current_stream())
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % period].replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        graphs[i % period].replay()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    return {"ms_per_step": ms, "value": tok_heads / (ms / 1e3), "graphs": period,
            "launch_overhead_us_per_layer": (eager_ms - ms) * 1e3 / n_layers}


def split_sweep(torch, np, hq, cfg, caches, q, out, n_ctx, stream, args):
    """Decode alone (no append) at each requested split count, caches rotated as in the step."""
    res = {}
    for S in [int(x) for x in args.split_sweep.split(",") if x.strip()]:
        nb = hq.decode_workspace_bytes(cfg, n_ctx, S)
        ws = torch.zeros((nb + 3) // 4, dtype=torch.float32, device=q.device)
        for i in range(args.warmup):
            caches[i % len(caches)].decode(q, n_ctx, out=out, out_dtype=hq.HEADQ_BF16, n_splits=S, ws=ws,
                                           stream=stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev[i][0].record(stream)
            caches[i % len(caches)].decode(q, n_ctx, out=out, out_dtype=hq.HEADQ_BF16, n_splits=S, ws=ws,
                                           stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        res[str(S) if S else "auto"] = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen7b_decode")
    ap.add_argument("--copies", type=int, default=2, help="cache copies rotated between steps")
    ap.add_argument("--splits", type=int, default=0, help="token splits per stream (0 = library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=32)
    ap.add_argument("--paged", action="store_true",
                    help="paged caches: every 32-token group in a page of shared pools, through a shuffled block table")
    ap.add_argument("--copy-probe", action="store_true", help="launch one 1 GiB device copy (counter scaling)")
    ap.add_argument("--value-protect", type=int, default=0,
                    help="A^2 value policy: corrected tokens per 32-token group (2-bit value workloads)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in HIP graphs (one per cache rotation) and replayed")
    ap.add_argument("--split-sweep", default="",
                    help="comma-separated split counts: also time the decode alone at each (0 = library choice)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "sharding over several GPUs is not built (the decode would shard over batch rows and KV heads "
              "with no exchange, each GPU running this kernel on its share).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_kv_cache_headq_amd as hq
    from workloads import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.workload in DIAG_WORKLOADS:
        run_diagnostics(args, hq, synth, torch, np)
        return
    if args.workload in PREFILL_WORKLOADS:
        run_prefill(args, hq, synth, torch, np)
        return
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    DT = {"f32": hq.HEADQ_F32, "bf16": hq.HEADQ_BF16}
    if args.value_protect and w.value_mode != "q2":
        print("bench.py: --value-protect needs a workload with 2-bit values", file=sys.stderr)
        sys.exit(2)
    cfg = hq.Config(head_dim=w.head_dim, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, batch=w.batch,
                    capacity=w.n_ctx, rank=w.rank, key_dtype=DT[w.key_dtype], value_dtype=DT[w.value_dtype],
                    value_mode=hq.HEADQ_V_DENSE if w.value_mode == "dense" else hq.HEADQ_V_Q2,
                    query_dtype=DT[w.query_dtype], value_protect=args.value_protect)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}

    # ---- inputs (seeded, synthetic), offline calibration
    qcal = synth.calibration_queries(w)
    t0 = time.perf_counter()
    U, _ = hq.headq_calibrate(cfg, qcal)
    a_dir = hq.headq_calibrate_mean(cfg, qcal) if args.value_protect else None
    calib_s = time.perf_counter() - t0
    append_only = w.name == "append_prefill"
    K = torch.from_numpy(synth.stack_streams(w, "keys", workers=16)).to(dev).to(tdt[w.key_dtype])
    V = None if append_only else torch.from_numpy(synth.stack_streams(w, "values", workers=16)).to(dev).to(
        tdt[w.value_dtype])
    q = torch.from_numpy(synth.decode_queries(w)).to(dev).to(tdt[w.query_dtype])
    n_layers = w.layers
    caches = []
    n_copies = max(args.copies, n_layers, 4 if append_only else 1)
    G = w.n_ctx // 32
    for i in range(n_copies):
        if args.paged:
            dc = hq.PagedDeviceCache(cfg, n_pages=w.batch * G, max_pages=G, device=dev)
            perm = np.random.default_rng(100 + i).permutation(w.batch * G).astype(np.int32)
            dc.block_table.copy_(torch.from_numpy(perm.reshape(w.batch, G)))
        else:
            dc = hq.DeviceCache(cfg, device=dev)
        dc.set_basis(U)
        if args.value_protect:
            dc.set_direction(a_dir)
        dc.append(K, V, 0)
        caches.append(dc)
    n_ctx = w.n_ctx
    last = n_ctx - 32
    k_new = K[:, :, last:]
    v_new = None if V is None else V[:, :, last:]
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    ws_bytes = hq.decode_workspace_bytes(cfg, n_ctx, args.splits)
    ws = torch.zeros((ws_bytes + 3) // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    copy_gbs = copy_ceiling(torch, dev, stream)
    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
    torch.cuda.synchronize()
    if append_only:
        # a prefill's keys are read once: rotate copies so the 256 MB MALL cannot serve them
        Ks = [K] + [K.clone() for _ in range(n_copies - 1)]
    else:
        del K, V

    # One step: decode workloads append the newest 32-token group of every stream and decode over
    # the whole context, once per layer (each layer its own cache); the prefill workload appends
    # the whole prefill.
    def run(i, marks=None, stream=stream):
        if append_only:
            dc = caches[i % len(caches)]
            if marks:
                marks[0].record(stream)
            dc.append(Ks[i % len(Ks)], None, 0, stream=stream)
            if marks:
                marks[1].record(stream)
            return
        for l in range(n_layers):
            dc = caches[(i * n_layers + l) % len(caches)]
            if marks:
                marks[2 * l].record(stream)
            dc.append(k_new, v_new, last, stream=stream)
            if marks:
                marks[2 * l + 1].record(stream)
            dc.decode(q, n_ctx, out=out, out_dtype=hq.HEADQ_BF16, n_splits=args.splits, ws=ws, stream=stream)
        if marks:
            marks[-1].record(stream)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()

    # ---- timed region: events on the stream the kernels run on
    n_marks = 2 if append_only else 2 * n_layers + 1
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_marks)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        run(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = np.array([m[0].elapsed_time(m[-1]) for m in ev])
    ms_per_step = float(step_ms.mean())
    if append_only:
        append_ms = step_ms
        decode_ms = None
    else:
        append_ms = np.array([[m[2 * l].elapsed_time(m[2 * l + 1]) for l in range(n_layers)] for m in ev])
        decode_ms = np.array([[m[2 * l + 1].elapsed_time(m[2 * l + 2]) for l in range(n_layers)] for m in ev])

    kinds = {"f32": "f32", "bf16": "bf16"}
    desc = {
        "tinyllama_decode": "TinyLlama-1.1B-shaped decode",
        "qwen7b_decode": "Qwen2.5-7B-shaped decode",
        "qwen14b_fullkv": "Qwen2.5-14B-shaped full-KV 2-bit decode",
        "append_prefill": "cache write of a prefill",
        "tiny": "tiny decode",
    }[w.name]
    config = {
        "workload": f"{w.name}: {desc}, Hq {w.n_q_heads}, Hkv {w.n_kv_heads}, d {w.head_dim}, batch {w.batch}, "
                    f"context {n_ctx}, 2-bit keys + rank-{w.rank} 4-bit side code"
                    + ("" if append_only else f", {w.value_mode} {kinds[w.value_dtype]} values")
                    + (f", {n_layers} layers" if n_layers > 1 else "")
                    + (", paged (shuffled 32-token pages)" if args.paged else "")
                    + (f", A^2 value policy ({args.value_protect} corrected tokens per group)"
                       if args.value_protect else ""),
        "batch": w.batch, "n_ctx": n_ctx, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
        "head_dim": w.head_dim, "rank": w.rank, "layers": n_layers,
        "step": ("headq_cache_append of the whole prefill (keys)" if append_only else
                 "per layer: append newest 32-token group + decode over the full context"),
        "cache_copies": len(caches), "n_splits": args.splits or "auto", "paged": bool(args.paged), "value_protect": args.value_protect,
    }
    result = {
        "metric": METRIC,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
    }
    if append_only:
        tok_heads = w.batch * w.n_kv_heads * n_ctx
        flops = 2 * w.rank * w.head_dim * tok_heads
        achieved = flops / (ms_per_step / 1e3) / 1e12
        result.update({
            "metric": "cache-append tokens·KV-heads/s, 1 GPU",
            "value": tok_heads / (ms_per_step / 1e3),
            "unit": "KV-head tokens/s",
            "roofline": {
                "bound": "alu", "kernel": "append_kernel (one launch)",
                "achieved": achieved, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / FP32_VECTOR_PEAK_TFLOPS, "traffic": traffic_per_launch(w.name),
                "peak_nonpacked": FP32_NONPACKED_PEAK_TFLOPS,
                "frac_nonpacked": achieved / FP32_NONPACKED_PEAK_TFLOPS,
                "algorithmic_flops_per_launch": flops,
                "hbm_gbs": append_bytes(w) * tok_heads / (ms_per_step / 1e3) / 1e9,
            },
        })
    else:
        tok_heads = w.batch * w.n_q_heads * n_ctx * n_layers
        per_tok = algorithmic_bytes_per_token_head(w, args.value_protect)
        alg_bytes = per_tok * w.batch * w.n_kv_heads * n_ctx
        dec_s = float(decode_ms.mean()) / 1e3
        achieved = alg_bytes / dec_s / 1e9
        mfma = w.value_mode == "q2" or w.value_dtype == "bf16"
        # counters were taken on contiguous caches without the value policy
        traffic = None if args.paged or args.value_protect else traffic_per_launch(w.name)
        result.update({
            "value": tok_heads / (ms_per_step / 1e3),
            "unit": "query-head cached tokens/s",
            "roofline": {
                "bound": "hbm",
                "kernel": ("headq_decode_attn (one launch: decode_mfma_kernel, splits merged in-kernel)" if mfma
                           else "headq_decode_attn (decode_split_kernel + decode_reduce_kernel)"),
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": traffic,
                "algorithmic_bytes_per_launch": alg_bytes,
                "bytes_per_token_kv_head": per_tok,
                "copy_ceiling_gbs": copy_gbs,
                "frac_of_copy_ceiling": achieved / copy_gbs,
            },
            "decode_ms": float(decode_ms.mean()),
            "decode_ms_p10_p90": [float(np.percentile(decode_ms, 10)), float(np.percentile(decode_ms, 90))],
            "append_ms": float(append_ms.mean()),
            "kv_head_tokens_per_s": w.batch * w.n_kv_heads * n_ctx * n_layers / (ms_per_step / 1e3),
        })
    if args.graph and not append_only:
        result["graph"] = time_graphs(torch, np, run, stream, len(caches), n_layers, args, tok_heads, ms_per_step)
    if args.split_sweep and not append_only:
        result["split_sweep_decode_ms"] = split_sweep(torch, np, hq, cfg, caches, q, out, n_ctx, stream, args)
    result["calibrate_s_host"] = calib_s
    result["wall_s_timed"] = wall
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        if append_only:
            result["cpu_baseline"] = append_cpu_baseline(w, U, threads)
        else:
            result["cpu_baseline"] = cpu_baseline(w, U, threads, min(args.cpu_rows, w.batch),
                                                  value_protect=args.value_protect, a_dir=a_dir)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
