"""GPU parity of paged caches: every packed array is a pool of pages (one 32-token group of all KV
heads), and a per-row block table says which page holds each group.

The rows are written at ragged, token-granular positions through a shuffled block table; after
each write the pools, gathered back through the table, must equal the oracle's contiguous cache
bit for bit, and a decode of the per-row lengths must match the oracle's logits and outputs.
Pages are an addressing change only, so the oracle's contiguous cache is the reference.
"""
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import oracle as orc
from workloads import synth

from .gpu_helpers import check_logits, check_out, compare_cache, config, say, to_device
from .helpers import VDT, VMODE, value_payload

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
PER_TOKEN = ("kcode", "scode", "ssc")          # one row per token: pages hold [Hkv][32][...]
PER_GROUP = ("kmeta", "v", "vcode", "vmeta", "vpidx", "vprot")  # one block per group: pages hold [Hkv][...]


def _gathered(pc, table, G):
    """Pools read back through the block table into the contiguous [B][Hkv][...] layout."""
    import torch
    idx = torch.as_tensor(table[:, :G], dtype=torch.long, device="cuda")
    B = idx.shape[0]
    out = SimpleNamespace(ktail=pc.ktail, vtail=pc.vtail)
    for name in PER_TOKEN + PER_GROUP:
        t = getattr(pc, name, None)
        if t is None:
            setattr(out, name, None)
            continue
        x = t[idx]                                   # [B][G][Hkv][...]
        x = x.transpose(1, 2).contiguous()           # [B][Hkv][G][...]
        if name in PER_TOKEN:
            x = x.reshape(B, x.shape[1], G * x.shape[3], *x.shape[4:])
        setattr(out, name, x)
    return out


def _run(w, B, cap, steps, out_bf16=False, n_splits=0, seed=11, value_protect=0, a_dir=None):
    import torch
    import quantized_kv_cache_headq_amd as hq
    G = cap // 32
    max_pages = G + 2                                # spare table columns are never read
    n_pages = B * G + 3                              # spare pages stay untouched
    rng = np.random.default_rng(seed)
    table = np.full((B, max_pages), 1 << 30, np.int32)
    table[:, :G] = rng.permutation(n_pages)[:B * G].reshape(B, G)
    say("paged", w.name, f"B={B} cap={cap} d={w.head_dim} r={w.rank} g={w.gqa} v={w.value_mode}/{w.value_dtype}",
        f"pages={n_pages} steps={steps} splits={n_splits}")
    U = orc.calibrate(synth.calibration_queries(w, n_cal=128), w.n_kv_heads, w.rank)[0] if w.rank else None
    Kf = synth.stack_streams(w, "keys", B, cap)
    Vf = synth.stack_streams(w, "values", B, cap)
    pc = hq.PagedDeviceCache(config(w, B, cap, value_protect), n_pages=n_pages, max_pages=max_pages)
    pc.block_table.copy_(torch.from_numpy(table))
    if w.rank:
        pc.set_basis(U)
    if value_protect:
        pc.set_direction(a_dir)
    oc = orc.empty_cache(B, w.n_kv_heads, cap, w.head_dim, w.rank, VMODE[w.value_mode], VDT[w.value_dtype],
                         key_dtype=VDT[w.key_dtype], base_bits=w.base_bits, value_protect=value_protect)
    lengths = np.array([(7 * b) % 32 for b in range(B)])  # rows start at different offsets
    for n_new in steps:
        K = np.stack([Kf[b, :, lengths[b]:lengths[b] + n_new] for b in range(B)])
        V = np.stack([Vf[b, :, lengths[b]:lengths[b] + n_new] for b in range(B)])
        rs = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        pc.append(to_device(K, w.key_dtype), to_device(V, w.value_dtype), 0, row_start=rs)
        for b in range(B):
            for h in range(w.n_kv_heads):
                orc.write_stream(oc, b, h, int(lengths[b]), K[b, h], value_payload(V[b, h], w),
                                 None if U is None else U[h], VMODE[w.value_mode], VDT[w.value_dtype],
                                 bits=w.base_bits, a_h=None if a_dir is None else a_dir[h])
        lengths = lengths + n_new
        compare_cache(_gathered(pc, table, G), oc)
        n_max = int(lengths.max())
        q = synth.decode_queries(w, position=n_max, batch=B)
        rl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        lg = torch.full((B, w.n_q_heads, n_max), float("nan"), device="cuda")
        out = pc.decode(to_device(q, w.query_dtype), n_max, out_dtype=hq.HEADQ_BF16 if out_bf16 else hq.HEADQ_F32,
                        logits_dbg=lg, n_splits=n_splits, row_len=rl)
        torch.cuda.synchronize()
        ref_l, ref_o = orc.decode(oc, q, U, n_max, 1.0, VMODE[w.value_mode], VDT[w.value_dtype], row_len=lengths)
        lg = lg.cpu().numpy()
        for b in range(B):
            check_logits(lg[b, :, :lengths[b]], ref_l[b, :, :lengths[b]])
        check_out(out.float().cpu().numpy(), ref_o, out_bf16)
    # the pages no row owns were never written
    owned = set(table[:, :G].ravel().tolist())
    spare = [p for p in range(n_pages) if p not in owned]
    for name in PER_TOKEN + PER_GROUP:
        t = getattr(pc, name, None)
        if t is not None:
            assert int((t[spare] != 0).sum()) == 0, name


STEPS = (40, 1, 30, 33, 2)


def test_paged_qwen7b_shape_dense_bf16_values():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2), 3, 160, STEPS)


def test_paged_fullkv_two_bit_values():
    _run(synth.scaled(W["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2), 3, 160, STEPS, out_bf16=True)


def test_paged_tinyllama_shape_d64():
    _run(synth.scaled(W["tinyllama_decode"], n_q_heads=16, n_kv_heads=2), 2, 160, STEPS)


def test_paged_tiny_f32_vector_kernel():
    _run(W["tiny"], 2, 160, STEPS)


def test_paged_with_splits():
    _run(synth.scaled(W["qwen7b_decode"], n_q_heads=14, n_kv_heads=2, rank=32), 2, 640, (300, 1, 240), n_splits=3)
