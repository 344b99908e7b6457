"""Host checks of the benchmark's bookkeeping (CPU only).

The roofline's algorithmic bytes per cached token and KV head are written as formulas in
bench.py; here they are derived independently from the cache format itself (the byte sizes of
the oracle's cache buffers divided by the tokens they hold) for every decode workload, with and
without the A^2 value policy. Also: the committed counter summaries still belong to the kernel
sources in the tree, and a request for more than one GPU is refused before any GPU work.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import oracle as orc
from workloads import synth

W = synth.WORKLOADS
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _format_bytes_per_token(w, value_protect=0):
    cap = 64
    vmode = 0 if w.value_mode == "dense" else 1
    vdt = 0 if w.value_dtype == "f32" else 1
    c = orc.empty_cache(1, 1, cap, w.head_dim, w.rank, vmode, vdt, value_protect=value_protect)
    names = ["kcode", "kmeta", "scode", "ssc", "v", "vcode", "vmeta", "vpidx", "vprot"]
    return sum(c[n].nbytes for n in names if n in c) / cap


@pytest.mark.parametrize("wname", ["tiny", "tinyllama_decode", "qwen7b_decode", "qwen14b_fullkv"])
def test_algorithmic_bytes_match_the_cache_format(wname):
    w = W[wname]
    assert bench.algorithmic_bytes_per_token_head(w) == _format_bytes_per_token(w)
    if w.value_mode == "q2":
        for p in (1, 2):
            assert bench.algorithmic_bytes_per_token_head(w, p) == _format_bytes_per_token(w, p)


def test_per_call_totals():
    """Bytes per decode call of the three decode workloads (token-KV-heads x bytes per token)."""
    totals = {"qwen7b_decode": 658_505_728, "tinyllama_decode": 42_467_328, "qwen14b_fullkv": 1_778_384_896}
    for name, total in totals.items():
        w = W[name]
        assert bench.algorithmic_bytes_per_token_head(w) * w.batch * w.n_kv_heads * w.n_ctx == total


def test_committed_counters_match_the_kernel_sources():
    for workload in bench.TRAFFIC:
        assert bench.traffic_per_launch(workload) is not None, workload


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr
    assert r.stdout == ""
