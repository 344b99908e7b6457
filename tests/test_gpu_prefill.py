"""GPU parity of headq_prefill_attn (chunked-prefill attention over the HeadQ cache).

The chunk's keys and values are appended first, as a chunked prefill does; every query token t
then attends the cached tokens 0 .. start + t of that cache. The oracle's prefill (its fp64
decode logits over the whole cache, cut at each position) runs on its own cache built from the
same generator arrays and pieces; logits and outputs must meet the decode's tolerances
(|dlogit| <= 1e-3 max(1, |s|); outputs 2e-3, plus half a bf16 ulp for bf16).
"""
import numpy as np
import pytest

from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import check_logits, check_out, gpu_cache, say, to_device
from .helpers import VDT, VMODE

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _queries(w, B, n_q, seed=5):
    rng = np.random.default_rng(seed)
    q = synth.decode_queries(w, batch=B * n_q, stream=seed).reshape(B, n_q, w.n_q_heads, w.head_dim)
    return np.ascontiguousarray(q)


def _run(w, B, start, n_q, out_bf16=False, kappa=1.0, cap=None, check_tokens=None):
    import torch
    import quantized_kv_cache_headq_amd as hq
    L = start + n_q
    say("prefill", w.name, f"B={B} start={start} n_q={n_q} d={w.head_dim} r={w.rank} g={w.gqa}",
        f"v={w.value_mode}/{w.value_dtype} kappa={kappa}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0] if w.rank else None
    cap = cap or (L + 31) // 32 * 32
    # the prefix as whole groups plus a tail, then the chunk (a token-granular append)
    n_full0 = start // 32 * 32
    pieces = [p for p in [(0, n_full0), (n_full0, start - n_full0), (start, n_q)] if p[1]]
    dc, K, V = gpu_cache(w, U, B, L, cap, pieces=pieces)
    q = _queries(w, B, n_q)
    lg = torch.full((B, n_q, w.n_q_heads, L), float("nan"), device="cuda")
    out = dc.prefill(to_device(q, w.query_dtype), start, out_dtype=hq.HEADQ_BF16 if out_bf16 else hq.HEADQ_F32,
                     corr_scale=kappa, logits_dbg=lg)
    torch.cuda.synchronize()
    lg = lg.cpu().numpy()
    out = out.float().cpu().numpy()
    oc = orc.empty_cache(B, w.n_kv_heads, cap, w.head_dim, w.rank, VMODE[w.value_mode], VDT[w.value_dtype],
                         key_dtype=VDT[w.key_dtype])
    from .helpers import value_payload
    for b in range(B):
        for h in range(w.n_kv_heads):
            for st, n in pieces:
                orc.write_stream(oc, b, h, st, K[b, h, st:st + n], value_payload(V[b, h, st:st + n], w),
                                 None if U is None else U[h], VMODE[w.value_mode], VDT[w.value_dtype])
    tokens = list(range(n_q)) if check_tokens is None else check_tokens
    ref_l, ref_o = orc.prefill(oc, q, U, start, kappa, VMODE[w.value_mode], VDT[w.value_dtype], tokens=tokens)
    for t in tokens:
        check_logits(lg[:, t, :, :start + t + 1], ref_l[:, t, :, :start + t + 1])
        check_out(out[:, t], ref_o[:, t], out_bf16)
        assert np.all(np.isnan(lg[:, t, :, start + t + 1:]))  # past the causal limit: untouched


def test_qwen7b_shape_chunk_ends_inside_a_group():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2), 2, 100, 37)


def test_whole_prompt_as_one_aligned_chunk():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2), 1, 0, 64)


def test_fullkv_two_bit_values_bf16_out():
    _run(synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2), 2, 64, 40, out_bf16=True)


def test_tinyllama_shape_d64():
    _run(synth.scaled(W["tinyllama_decode"], n_q_heads=16, n_kv_heads=2), 2, 33, 50)


def test_rank32_wrong_sign_half_scale_and_rank0():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1, rank=32), 1, 70, 26, kappa=-1.0)
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1), 1, 70, 26, kappa=0.5)
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1, rank=0), 1, 70, 26)


def test_sixteen_heads_few_tokens():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=16, n_kv_heads=1, rank=8), 2, 200, 5)


def test_single_token_chunk():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=7, n_kv_heads=1), 2, 95, 1)


def test_long_prefix_sampled_tokens():
    """A 4096-token prefix and a 256-token chunk (several workgroups per stream, every column
    walking 130+ groups); the oracle checks a sample of query tokens."""
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2), 1, 4096, 256,
         check_tokens=[0, 1, 63, 64, 127, 200, 255])


def test_paged_cache_prefill():
    """The same chunked prefill through a shuffled block table (pages of shared pools)."""
    import torch
    import quantized_kv_cache_headq_amd as hq
    from .gpu_helpers import config
    from .helpers import value_payload
    w = synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2)
    B, start, n_q, cap = 2, 70, 50, 128
    L = start + n_q
    say("prefill-paged", w.name, f"B={B} start={start} n_q={n_q}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0]
    G = cap // 32
    rng = np.random.default_rng(4)
    table = rng.permutation(B * G + 2)[:B * G].reshape(B, G).astype(np.int32)
    pc = hq.PagedDeviceCache(config(w, B, cap), n_pages=B * G + 2, max_pages=G)
    pc.block_table.copy_(torch.from_numpy(table))
    pc.set_basis(U)
    K = synth.stack_streams(w, "keys", B, L)
    V = synth.stack_streams(w, "values", B, L)
    pieces = [(0, 64), (64, 6), (70, 50)]
    oc = orc.empty_cache(B, w.n_kv_heads, cap, w.head_dim, w.rank, 0, 1, key_dtype=1)
    for st, n in pieces:
        pc.append(to_device(K[:, :, st:st + n], w.key_dtype), to_device(V[:, :, st:st + n], w.value_dtype), st)
        for b in range(B):
            for h in range(w.n_kv_heads):
                orc.write_stream(oc, b, h, st, K[b, h, st:st + n], value_payload(V[b, h, st:st + n], w), U[h], 0, 1)
    q = _queries(w, B, n_q)
    lg = torch.full((B, n_q, w.n_q_heads, L), float("nan"), device="cuda")
    out = pc.prefill(to_device(q, w.query_dtype), start, logits_dbg=lg)
    torch.cuda.synchronize()
    lg, out = lg.cpu().numpy(), out.float().cpu().numpy()
    tokens = [0, 10, 25, 49]
    ref_l, ref_o = orc.prefill(oc, q, U, start, 1.0, 0, 1, tokens=tokens)
    for t in tokens:
        check_logits(lg[:, t, :, :start + t + 1], ref_l[:, t, :, :start + t + 1])
        check_out(out[:, t], ref_o[:, t], False)
