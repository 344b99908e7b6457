"""Benchmark of the HeadQ decode hot path on one MI355X.

python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload qwen7b_decode] [--no-cpu-baseline]

One step = one decode step of the workload through libheadq: headq_cache_append of the newest
32-token group of every (b, h) stream, then headq_decode_attn over the whole context. The
calibration (host PCA) runs once before timing, as the method prescribes (offline), and is
reported separately. Inputs are seeded synthetic tensors resident in HBM before timing starts;
several cache copies are rotated so the 256 MB MALL cannot hold the working set.

Prints one JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn cached tokens·heads/s + achieved HBM GB/s (% of peak), 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_qwen7b_traffic.json")
DECODE_SRC = os.path.join(ROOT, "quantized_kv_cache_headq_amd", "csrc", "decode_mfma.hip")


def algorithmic_bytes_per_token_head(w) -> int:
    """Bytes the method must move per cached token per KV head (keys, side code, values)."""
    d, r = w.head_dim, w.rank
    k = d // 4 + d // 8 + r // 2 + (2 if r else 0)  # 2-bit codes, fp16 step/zero per 32 tokens, nibbles, sigma
    if w.value_mode == "dense":
        v = d * (4 if w.value_dtype == "f32" else 2)
    else:
        v = d // 4 + d // 8  # 2-bit codes, fp16 step/zero per 32 channels
    return k + v


def source_sha() -> str:
    return hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()[:16]


def traffic_per_launch():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, or None when the
    decode kernel source changed since the counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != source_sha():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, U, threads: int, rows: int, cpu_seconds: float = 15.0):
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
        oc = orc.empty_cache(1, w.n_kv_heads, w.n_ctx, w.head_dim, w.rank, vmode, vdt)
        for h in range(w.n_kv_heads):
            k = synth.keys(w, b, h)
            v = synth.values(w, b, h)
            if vmode == 0 and vdt == 1:
                v = (v.view(np.uint32) >> 16).astype(np.uint16)
            orc.write_stream(oc, 0, h, 0, k, v, U[h], vmode, vdt)
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
    return {"value": n / wall, "unit": "query-head cached tokens/s", "cores": min(threads, rows), "kind": "oracle",
            "sample": f"fp64 oracle decode of {rows} of {w.batch} batch rows x {w.n_q_heads} query heads x "
                      f"{w.n_ctx} tokens, {passes} passes ({wall:.2f} s wall, {cpu:.1f} s CPU)"}


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
    ap.add_argument("--copy-probe", action="store_true", help="launch one 1 GiB device copy (counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "multi-GPU sharding is described in DESIGN.md but not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_kv_cache_headq_amd as hq
    from workloads import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    DT = {"f32": hq.HEADQ_F32, "bf16": hq.HEADQ_BF16}
    cfg = hq.Config(head_dim=w.head_dim, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, batch=w.batch,
                    capacity=w.n_ctx, rank=w.rank, key_dtype=DT[w.key_dtype], value_dtype=DT[w.value_dtype],
                    value_mode=hq.HEADQ_V_DENSE if w.value_mode == "dense" else hq.HEADQ_V_Q2,
                    query_dtype=DT[w.query_dtype])
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}

    # ---- inputs (seeded, synthetic), offline calibration
    qcal = synth.calibration_queries(w)
    t0 = time.perf_counter()
    U, _ = hq.headq_calibrate(cfg, qcal)
    calib_s = time.perf_counter() - t0
    K = torch.from_numpy(synth.stack_streams(w, "keys", workers=16)).to(dev).to(tdt[w.key_dtype])
    V = torch.from_numpy(synth.stack_streams(w, "values", workers=16)).to(dev).to(tdt[w.value_dtype])
    q = torch.from_numpy(synth.decode_queries(w)).to(dev).to(tdt[w.query_dtype])
    caches = []
    for _ in range(args.copies):
        dc = hq.DeviceCache(cfg, device=dev)
        dc.set_basis(U)
        dc.append(K, V, 0)
        caches.append(dc)
    n_ctx = w.n_ctx
    last = n_ctx - 32
    k_new, v_new = K[:, :, last:], V[:, :, last:]
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    ws_bytes = hq.decode_workspace_bytes(cfg, n_ctx, args.splits)
    ws = torch.zeros((ws_bytes + 3) // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
    torch.cuda.synchronize()
    del K, V

    def step(i):
        dc = caches[i % len(caches)]
        dc.append(k_new, v_new, last, stream=stream)
        dc.decode(q, n_ctx, out=out, out_dtype=hq.HEADQ_BF16, n_splits=args.splits, ws=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: events on the stream the kernels run on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        dc = caches[i % len(caches)]
        e0, e1, e2 = ev[i]
        e0.record(stream)
        dc.append(k_new, v_new, last, stream=stream)
        e1.record(stream)
        dc.decode(q, n_ctx, out=out, out_dtype=hq.HEADQ_BF16, n_splits=args.splits, ws=ws, stream=stream)
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    append_ms = np.array([e0.elapsed_time(e1) for e0, e1, _ in ev])
    decode_ms = np.array([e1.elapsed_time(e2) for _, e1, e2 in ev])
    step_ms = np.array([e0.elapsed_time(e2) for e0, _, e2 in ev])
    ms_per_step = float(step_ms.mean())

    tok_heads = w.batch * w.n_q_heads * n_ctx
    value = tok_heads / (ms_per_step / 1e3)
    per_tok = algorithmic_bytes_per_token_head(w)
    alg_bytes = per_tok * w.batch * w.n_kv_heads * n_ctx
    dec_s = float(decode_ms.mean()) / 1e3
    achieved = alg_bytes / dec_s / 1e9
    traffic = traffic_per_launch()

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "query-head cached tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: Qwen2.5-7B-shaped decode, Hq {w.n_q_heads}, Hkv {w.n_kv_heads}, d {w.head_dim}, "
                        f"batch {w.batch}, context {n_ctx}, 2-bit keys + rank-{w.rank} 4-bit side code, "
                        f"{w.value_mode} {w.value_dtype} values" if w.name == "qwen7b_decode" else w.name,
            "batch": w.batch, "n_ctx": n_ctx, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "rank": w.rank, "io": "bf16 queries/keys/values, bf16 output",
            "step": "append newest 32-token group + decode over the full context",
            "cache_copies": len(caches), "n_splits": args.splits or "auto",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "headq_decode_attn (one launch: decode_mfma_kernel, splits merged in-kernel)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes,
            "bytes_per_token_kv_head": per_tok,
        },
        "decode_ms": float(decode_ms.mean()),
        "decode_ms_p10_p90": [float(np.percentile(decode_ms, 10)), float(np.percentile(decode_ms, 90))],
        "append_ms": float(append_ms.mean()),
        "kv_head_tokens_per_s": w.batch * w.n_kv_heads * n_ctx / (ms_per_step / 1e3),
        "calibrate_s_host": calib_s,
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        result["cpu_baseline"] = cpu_baseline(w, U, threads, min(args.cpu_rows, w.batch))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
