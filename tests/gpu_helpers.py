"""Helpers for the GPU tests: build libheadq caches from the seeded workloads and compare them
with the oracle's."""
from __future__ import annotations

import sys

import numpy as np

from oracle import oracle as orc
from workloads import synth

from .helpers import VDT, VMODE, oracle_cache, value_payload

DT = {"f32": 0, "bf16": 1}


def say(*a):
    """Name the case on stdout before each GPU step (flushed)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def config(w: synth.Workload, batch=None, cap=None, value_protect=0):
    import quantized_kv_cache_headq_amd as hq
    return hq.Config(head_dim=w.head_dim, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                     batch=w.batch if batch is None else batch, capacity=w.n_ctx if cap is None else cap,
                     rank=w.rank, key_dtype=DT[w.key_dtype], value_dtype=DT[w.value_dtype],
                     value_mode=VMODE[w.value_mode], query_dtype=DT[w.query_dtype], base_bits=w.base_bits,
                     value_protect=value_protect)


def torch_dtype(name):
    import torch
    return torch.float32 if name == "f32" else torch.bfloat16


def to_device(x_f32: np.ndarray, dtype_name: str):
    """f32 numpy holding values already rounded to dtype_name -> device tensor (exact)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to("cuda").to(torch_dtype(dtype_name))


def gpu_cache(w: synth.Workload, U, batch=None, T=None, cap=None, K=None, V=None, pieces=None, value_protect=0,
              a_dir=None):
    """Allocate a DeviceCache, set U (and the A^2 value policy's direction a_dir when
    value_protect > 0), and append the workload's keys/values (optionally in pieces
    [(start, n), ...]). Returns (DeviceCache, K f32 numpy, V f32 numpy)."""
    import quantized_kv_cache_headq_amd as hq
    B = w.batch if batch is None else batch
    T = w.n_ctx if T is None else T
    cap = T if cap is None else cap
    if K is None:
        K = synth.stack_streams(w, "keys", B, T)
    if V is None:
        V = synth.stack_streams(w, "values", B, T)
    dc = hq.DeviceCache(config(w, B, cap, value_protect))
    if w.rank:
        dc.set_basis(U)
    if value_protect:
        dc.set_direction(a_dir)
    Kd = to_device(K, w.key_dtype)
    Vd = to_device(V, w.value_dtype)
    for start, n in (pieces or [(0, T)]):
        dc.append(Kd[:, :, start:start + n], Vd[:, :, start:start + n], start)
    return dc, K, V


def host(t, view_u16=False):
    import torch
    x = t.detach().cpu()
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16)
    a = x.numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def compare_cache(dc, oc, streams=None):
    """Bit-exact comparison of every cache buffer (optionally only some (b, h) streams)."""
    pairs = [("kcode", dc.kcode), ("kmeta", dc.kmeta), ("scode", dc.scode), ("ssc", dc.ssc), ("v", dc.v),
             ("vcode", dc.vcode), ("vmeta", dc.vmeta), ("ktail", dc.ktail), ("vtail", dc.vtail),
             ("vpidx", getattr(dc, "vpidx", None)), ("vprot", getattr(dc, "vprot", None))]
    for name, t in pairs:
        if t is None or name not in oc or oc[name].size == 0:
            continue
        g = host(t)
        o = oc[name]
        if name == "vpidx":  # one little-endian word per group: the oracle keeps its four bytes
            g, o = g.view(np.uint32), np.ascontiguousarray(o).view(np.uint32)[..., 0]
        if streams is not None:
            g = np.stack([g[b, h] for b, h in streams])
            o = np.stack([o[b, h] for b, h in streams])
        if g.dtype == np.float32:
            g, o = g.view(np.uint32), o.view(np.uint32)
        assert g.shape == o.shape, (name, g.shape, o.shape)
        bad = np.argwhere(g != o)
        assert bad.size == 0, f"{name}: {len(bad)} mismatching elements, first at {bad[:3].tolist()}"


def check_logits(gpu_logits: np.ndarray, ref: np.ndarray):
    """|delta| <= 1e-3 * max(1, |s_ref|) in natural-log units."""
    tol = 1e-3 * np.maximum(1.0, np.abs(ref))
    err = np.abs(gpu_logits.astype(np.float64) - ref)
    worst = np.max(err / tol)
    assert worst <= 1.0, f"logit error {worst:.3f} x tolerance (max abs {err.max():.3e})"


def check_out(gpu_out: np.ndarray, ref: np.ndarray, bf16: bool):
    """|delta| <= 2e-3 (f32 output) or 2e-3 + half a bf16 ulp of the reference (bf16 output)."""
    tol = np.full(ref.shape, 2e-3)
    if bf16:
        e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-30)))
        tol = tol + 0.5 * 2.0 ** (e - 7)
    err = np.abs(gpu_out.astype(np.float64) - ref)
    worst = np.max(err / tol)
    assert worst <= 1.0, f"output error {worst:.3f} x tolerance (max abs {err.max():.3e})"


def oracle_for(w, U, K, V, cap):
    """Oracle cache from the same f32 arrays (keys/values are generator outputs, never GPU ones)."""
    B, H, T, _ = K.shape
    kv = {(b, h): (K[b, h], V[b, h]) for b in range(B) for h in range(H)}
    oc, _ = oracle_cache(w, U, batch=B, n_tok=T, cap=cap, kv=kv)
    return oc


def oracle_pieces(w, U, K, V, cap, pieces):
    """The oracle's cache of the same generator (or hand-built) arrays, written in the same pieces
    [(start, n), ...] as the GPU cache (tokens past the last whole group go to the tails)."""
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


def decode_gpu(dc, w, q_f32, n_ctx, out_bf16=False, corr=1.0, n_splits=0, logits=True):
    import torch
    import quantized_kv_cache_headq_amd as hq
    qd = to_device(q_f32, w.query_dtype)
    lg = torch.full((q_f32.shape[0], w.n_q_heads, n_ctx), float("nan"), device="cuda") if logits else None
    out = dc.decode(qd, n_ctx, out_dtype=hq.HEADQ_BF16 if out_bf16 else hq.HEADQ_F32, corr_scale=corr,
                    logits_dbg=lg, n_splits=n_splits)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    return (lg.cpu().numpy() if logits else None), o
