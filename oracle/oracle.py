"""Python binding of the CPU oracle (``headq_oracle.c``) — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may import this
module. The product library never imports it and shares no code with it.

What it computes is cited in ``headq_oracle.c`` (HeadQ technical summary, §3 steps 1-3; §1 and
§2.2 for the readout). This file only marshals numpy arrays into the C calls and assembles the
per-stream results into the cache format.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "headq_oracle.c"
_LIB = _HERE / "liboracle.so"
GROUP = 32

_CFLAGS = ["-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> Path:
    """Compile the oracle with gcc (no contraction, IEEE semantics)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.run(["gcc", *_CFLAGS, str(_SRC), "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(str(_LIB))
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        for name in ("orc_f32_to_f16_array", "orc_f16_to_f32_array", "orc_f32_to_bf16_array"):
            getattr(L, name).argtypes = [P, P, I64]
            getattr(L, name).restype = None
        L.orc_calibrate.argtypes = [I, I, I, I64, I, I, P, P, P]
        L.orc_encode_keys.argtypes = [I, I, I, I, I64, P, P, P, P, P, P, P, P, P]
        L.orc_quantize_values.argtypes = [I, I, I64, P, P, P, P]
        L.orc_pack_kcode.argtypes = [I, I64, P, P]
        L.orc_pack_kcode4.argtypes = [I, I64, P, P]
        L.orc_pack_kmeta.argtypes = [I, I64, P, P, P]
        L.orc_pack_scode.argtypes = [I, I64, P, P]
        L.orc_pack_vdense.argtypes = [I, I64, I, P, P]
        L.orc_pack_vcode.argtypes = [I, I64, P, P]
        L.orc_pack_vmeta.argtypes = [I, I64, P, P, P]
        L.orc_decode.argtypes = [I, I, I, I, I, I, I, I64, I64, P, P, P, P, P, P, P, I, P, P, P, P, D, I, I, P, P, I,
                                 I, P, P]
        L.orc_value_rows.argtypes = [I, I, I, I, I64, I64, P, P, P, P, I, I, P, I, P, P]
        L.orc_policy_scale.restype = ctypes.c_float
        L.orc_policy_scale.argtypes = [I]
        L.orc_mean_query.argtypes = [I, I, I, I64, P, P]
        L.orc_value_policy.argtypes = [I, I, I64, P, P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


# --------------------------------------------------------------------------------------------
# number formats

def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_f16_array(_p(x), _p(out), x.size)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().orc_f16_to_f32_array(_p(h), _p(out), h.size)
    return out


def f32_to_bf16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_array(_p(x), _p(out), x.size)
    return out


def bf16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------------
# calibration, encode, decode

def calibrate(q_cal, n_kv_heads: int, rank: int, centered: bool = False):
    """Per-KV-head query PCA. q_cal: f32 [Hq][n_cal][d] -> (U f32 [Hkv][d][r], eig f64 [Hkv][r])."""
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    hq, n_cal, d = q.shape
    U = np.zeros((n_kv_heads, d, rank), dtype=np.float32)
    eig = np.zeros((n_kv_heads, rank), dtype=np.float64)
    _check(lib().orc_calibrate(d, hq, n_kv_heads, n_cal, rank, int(centered), _p(q), _p(U), _p(eig)),
           "calibrate")
    return U, eig


def encode_keys(k, U, bits: int = 2, side_bits: int = 4):
    """Encode one key stream. k: f32 [T][d], U: f32 [d][r] (or None for r = 0)."""
    k = np.ascontiguousarray(k, dtype=np.float32)
    T, d = k.shape
    r = 0 if U is None else U.shape[1]
    Uc = None if U is None else np.ascontiguousarray(U, dtype=np.float32)
    out = dict(
        codes=np.zeros((T, d), np.uint8), scale=np.zeros((T // GROUP, d), np.uint16),
        zero=np.zeros((T // GROUP, d), np.uint16), zc=np.zeros((T, max(r, 1)), np.int8)[:, :r].copy(),
        sigma=np.zeros(T, np.uint16), resid=np.zeros((T, d), np.float32), proj=np.zeros((T, max(r, 1)), np.float32),
    )
    zc_buf = out["zc"] if r else None
    _check(lib().orc_encode_keys(d, r, bits, side_bits, T, _p(k), _p(Uc), _p(out["codes"]), _p(out["scale"]),
                                 _p(out["zero"]), _p(zc_buf), _p(out["sigma"]), _p(out["resid"]), _p(out["proj"])),
           "encode_keys")
    out["proj"] = out["proj"][:, :r]
    return out


def mean_query(q_cal, n_kv_heads: int):
    """Mean calibration query per KV head (the A^2 value policy's direction): f32 [Hq][n_cal][d]
    -> f32 [Hkv][d]."""
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    hq, n_cal, d = q.shape
    a = np.zeros((n_kv_heads, d), np.float32)
    _check(lib().orc_mean_query(d, hq, n_kv_heads, n_cal, _p(q), _p(a)), "mean_query")
    return a


def value_policy(k, v, a_h, n_prot: int):
    """The A^2 value policy over whole groups of one stream: k, v f32 [T][d], a_h f32 [d]. Returns
    dict(idx u8 [T/32][4], delta bf16 bits [T/32][P][d], prio f64 [T], and the 2-bit value
    quantizer's codes/scale/zero)."""
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    a_h = np.ascontiguousarray(a_h, np.float32)
    T, d = v.shape
    vq = quantize_values(v, 2)
    idx = np.zeros((T // GROUP, 4), np.uint8)
    delta = np.zeros((T // GROUP, n_prot, d), np.uint16)
    prio = np.zeros(T, np.float64)
    _check(lib().orc_value_policy(d, n_prot, T, _p(k), _p(v), _p(a_h), _p(vq["codes"]), _p(vq["scale"]),
                                  _p(vq["zero"]), _p(idx), _p(delta), _p(prio)), "value_policy")
    return dict(idx=idx, delta=delta, prio=prio, **vq)


def quantize_values(v, bits: int = 2):
    v = np.ascontiguousarray(v, dtype=np.float32)
    T, d = v.shape
    codes = np.zeros((T, d), np.uint8)
    scale = np.zeros((T, d // GROUP), np.uint16)
    zero = np.zeros((T, d // GROUP), np.uint16)
    _check(lib().orc_quantize_values(d, bits, T, _p(v), _p(codes), _p(scale), _p(zero)), "quantize_values")
    return dict(codes=codes, scale=scale, zero=zero)


def empty_cache(B, Hkv, cap, d, r, value_mode, value_dtype, key_dtype=None, base_bits=2, value_protect=0):
    """Zero-filled buffers of the cache format (numpy, host). With key_dtype given, the dense tails
    of the unfinished last group are included: ktail / vtail [B][Hkv][32][d] in the key / value
    dtype (f32, or bfloat16 bit patterns). base_bits 2 packs four key codes per byte; 3 and 4 one
    code per nibble (kcode rows of d/2 bytes). value_protect P > 0 (2-bit values): the A^2 value
    policy's vpidx u8 [B][Hkv][cap/32][4] and vprot bf16 bits [B][Hkv][cap/32][P][d]; write_stream
    then needs the direction a_h of each head."""
    c = dict(
        kcode=np.zeros((B, Hkv, cap, d // 4 if base_bits == 2 else d // 2), np.uint8),
        kmeta=np.zeros((B, Hkv, cap // GROUP, 2, d), np.uint16),
        scode=np.zeros((B, Hkv, cap, max(r // 2, 0)), np.uint8),
        ssc=np.zeros((B, Hkv, cap), np.uint16),
    )
    if value_mode == 0:
        dt = np.float32 if value_dtype == 0 else np.uint16
        c["v"] = np.zeros((B, Hkv, cap // GROUP, d, GROUP), dt)
    else:
        c["vcode"] = np.zeros((B, Hkv, cap // GROUP, d * 8), np.uint8)
        c["vmeta"] = np.zeros((B, Hkv, cap // GROUP, 2, d // GROUP, GROUP), np.uint16)
        if value_protect:
            c["vpidx"] = np.zeros((B, Hkv, cap // GROUP, 4), np.uint8)
            c["vprot"] = np.zeros((B, Hkv, cap // GROUP, value_protect, d), np.uint16)
    if key_dtype is not None:
        c["ktail"] = np.zeros((B, Hkv, GROUP, d), np.float32 if key_dtype == 0 else np.uint16)
        c["vtail"] = np.zeros((B, Hkv, GROUP, d), np.float32 if value_dtype == 0 else np.uint16)
    return c


def _to_tail(x_f32_or_bits, tail):
    """Rows for a dense tail: f32 tails take f32 values, bf16 tails bit patterns (uint16)."""
    if tail.dtype == np.float32:
        return np.asarray(x_f32_or_bits, np.float32)
    x = np.asarray(x_f32_or_bits)
    return x if x.dtype == np.uint16 else f32_to_bf16_bits(x)


def _from_tail(rows, as_bits):
    """Tail rows back as f32 values, or as bf16 bit patterns when as_bits."""
    if rows.dtype == np.float32:
        return rows.copy()
    return rows.copy() if as_bits else bf16_bits_to_f32(rows)


def write_stream(cache, b, h, start, k, v, U_h, value_mode, value_dtype, bits=2, side_bits=4, a_h=None):
    """Append tokens [start, start + n) of one (b, h) stream (the cache write of the summary's §3
    step 2, one token at a time or in any run). Every group that is whole once these tokens are in
    is encoded; the tokens of an unfinished last group are kept exactly in the dense tails. Tokens
    of the first group that precede `start` must already be in the tail (earlier appends).

    k: f32 [n][d] keys (exact widening of the stored key dtype)
    v: [n][d] values (f32 array for dtype 0, bf16 bit patterns uint16 for dtype 1, f32 for 2-bit)
    a_h: f32 [d], the A^2 value policy's direction (caches with vprot)
    Returns the unpacked encode result of the whole groups (None if there are none)."""
    n, d = k.shape
    if start % GROUP == 0 and n % GROUP == 0:
        return _write_groups(cache, b, h, start, k, v, U_h, value_mode, value_dtype, bits, side_bits, a_h)
    g0 = start // GROUP
    head = start - g0 * GROUP
    kt, vt = cache["ktail"][b, h], cache["vtail"][b, h]
    v_bits = v is not None and value_mode == 0 and value_dtype == 1
    k_all = np.concatenate([_from_tail(kt[:head], False), np.asarray(k, np.float32)])
    v_all = None
    if v is not None:
        v_all = np.concatenate([_from_tail(vt[:head], v_bits), np.asarray(v, np.uint16 if v_bits else np.float32)])
    n_whole = (start + n) // GROUP - g0
    enc = None
    if n_whole > 0:
        m = n_whole * GROUP
        enc = _write_groups(cache, b, h, g0 * GROUP, k_all[:m], None if v_all is None else v_all[:m], U_h,
                            value_mode, value_dtype, bits, side_bits, a_h)
    rest = len(k_all) - n_whole * GROUP
    if rest:
        kt[:rest] = _to_tail(k_all[n_whole * GROUP:], kt)
        if v_all is not None:
            vt[:rest] = _to_tail(v_all[n_whole * GROUP:], vt)
    return enc


def _write_groups(cache, b, h, start, k, v, U_h, value_mode, value_dtype, bits, side_bits, a_h=None):
    """Encode whole groups (start and n multiples of 32) into the packed arrays."""
    n, d = k.shape
    r = 0 if U_h is None else U_h.shape[1]
    enc = encode_keys(k, U_h, bits, side_bits)
    L = lib()
    g0, g1 = start // GROUP, (start + n) // GROUP
    if bits == 2:
        kc = np.zeros((n, d // 4), np.uint8)
        _check(L.orc_pack_kcode(d, n, _p(enc["codes"]), _p(kc)), "pack_kcode")
    else:
        kc = np.zeros((n, d // 2), np.uint8)
        _check(L.orc_pack_kcode4(d, n, _p(enc["codes"]), _p(kc)), "pack_kcode4")
    cache["kcode"][b, h, start:start + n] = kc
    km = np.zeros((n // GROUP, 2, d), np.uint16)
    _check(L.orc_pack_kmeta(d, n, _p(enc["scale"]), _p(enc["zero"]), _p(km)), "pack_kmeta")
    cache["kmeta"][b, h, g0:g1] = km
    if r:
        sc = np.zeros((n, r // 2), np.uint8)
        _check(L.orc_pack_scode(r, n, _p(np.ascontiguousarray(enc["zc"])), _p(sc)), "pack_scode")
        cache["scode"][b, h, start:start + n] = sc
    cache["ssc"][b, h, start:start + n] = enc["sigma"]
    if v is not None:
        if value_mode == 0:
            src = np.ascontiguousarray(v)
            eb = src.dtype.itemsize
            dst = np.zeros((n // GROUP, d, GROUP), src.dtype)
            _check(L.orc_pack_vdense(d, n, eb, _p(src), _p(dst)), "pack_vdense")
            cache["v"][b, h, g0:g1] = dst
        else:
            vq = quantize_values(v, 2)  # 2-bit values whatever the key base bits
            vc = np.zeros((n // GROUP, d * 8), np.uint8)
            _check(L.orc_pack_vcode(d, n, _p(vq["codes"]), _p(vc)), "pack_vcode")
            cache["vcode"][b, h, g0:g1] = vc
            vm = np.zeros((n // GROUP, 2, d // GROUP, GROUP), np.uint16)
            _check(L.orc_pack_vmeta(d, n, _p(vq["scale"]), _p(vq["zero"]), _p(vm)), "pack_vmeta")
            cache["vmeta"][b, h, g0:g1] = vm
            if "vprot" in cache:
                if a_h is None:
                    raise ValueError("a cache with the A^2 value policy needs the direction a_h")
                pol = value_policy(k, v, a_h, cache["vprot"].shape[3])
                cache["vpidx"][b, h, g0:g1] = pol["idx"]
                cache["vprot"][b, h, g0:g1] = pol["delta"]
    return enc


def decode(cache, q, U, n_ctx, kappa=1.0, value_mode=0, value_dtype=1, b_range=None, want_logits=True,
           row_len=None):
    """fp64 decode attention from the packed cache.

    q: f32 [B][Hq][d]; U: f32 [Hkv][d][r] (or None). Returns (logits f64 [B][Hq][n_ctx] natural-log
    units or None, out f64 [B][Hq][d]); rows outside b_range stay zero. row_len: optional per-row
    token counts (each <= n_ctx); a row's logits past its length stay zero."""
    if row_len is not None:
        B = q.shape[0]
        out = np.zeros((B, q.shape[1], q.shape[2]), np.float64)
        logits = np.zeros((B, q.shape[1], n_ctx), np.float64) if want_logits else None
        for b in range(B):
            lg, o = decode(cache, q, U, int(row_len[b]), kappa, value_mode, value_dtype, (b, b + 1), want_logits)
            out[b] = o[b]
            if want_logits:
                logits[b, :, :int(row_len[b])] = lg[b]
        return logits, out
    kcode = np.ascontiguousarray(cache["kcode"])
    B, Hkv, cap, _ = kcode.shape
    q = np.ascontiguousarray(q, dtype=np.float32)
    _, Hq, d = q.shape
    r = 0 if U is None else U.shape[2]
    b0, b1 = (0, B) if b_range is None else b_range
    out = np.zeros((B, Hq, d), np.float64)
    logits = np.zeros((B, Hq, n_ctx), np.float64) if want_logits else None
    arrs = {k: np.ascontiguousarray(val) for k, val in cache.items()}
    Uc = None if U is None else np.ascontiguousarray(U, dtype=np.float32)
    kt = arrs.get("ktail")
    key_dtype = 0 if kt is None or kt.dtype == np.float32 else 1
    layout_bits = 2 if kcode.shape[3] * 4 == d else 4  # packing only: the levels do not enter k_hat
    n_prot = arrs["vprot"].shape[3] if "vprot" in arrs else 0
    _check(lib().orc_decode(d, Hq, Hkv, r, value_mode, value_dtype, B, cap, n_ctx, _p(arrs["kcode"]),
                            _p(arrs["kmeta"]), _p(arrs["scode"]) if r else None, _p(arrs["ssc"]) if r else None,
                            _p(arrs.get("v")), _p(arrs.get("vcode")), _p(arrs.get("vmeta")), key_dtype, _p(kt),
                            _p(arrs.get("vtail")), _p(Uc), _p(q), float(kappa), b0, b1, _p(logits), _p(out),
                            layout_bits, n_prot, _p(arrs.get("vpidx")), _p(arrs.get("vprot"))),
           "decode")
    return logits, out


def value_rows(cache, b, h, n_ctx, value_mode=0, value_dtype=1):
    """Value rows of stream (b, h) as the cache holds them: f64 [n_ctx][d] (dense as stored,
    2-bit as code * s + z, the unfinished group from the tail)."""
    arrs = {k: np.ascontiguousarray(val) for k, val in cache.items()}
    B, Hkv, cap, _ = arrs["kcode"].shape
    d = arrs["kmeta"].shape[-1]
    out = np.zeros((n_ctx, d), np.float64)
    n_prot = arrs["vprot"].shape[3] if "vprot" in arrs else 0
    _check(lib().orc_value_rows(d, value_mode, value_dtype, Hkv, cap, n_ctx, _p(arrs.get("v")), _p(arrs.get("vcode")),
                                _p(arrs.get("vmeta")), _p(arrs.get("vtail")), b, h, _p(out), n_prot,
                                _p(arrs.get("vpidx")), _p(arrs.get("vprot"))), "value_rows")
    return out


def prefill(cache, q, U, start, kappa=1.0, value_mode=0, value_dtype=1, tokens=None):
    """Chunked-prefill attention over the packed cache (the summary's §3 step 3 read, per query
    token): the cache holds tokens [0, start + n_q) — whole groups packed, the unfinished group
    exact in the tails — and query token t, at position start + t, attends tokens 0 .. start + t of
    that cache (causal), with the corrected logits of the oracle decode over the whole cache and
    the cache's value rows.

    q: f32 [B][n_q][Hq][d]. Returns (logits f64 [B][n_q][Hq][start + n_q], zero past each token's
    causal limit; out f64 [B][n_q][Hq][d]); with `tokens`, only those query tokens are computed
    (the others stay zero)."""
    q = np.ascontiguousarray(q, np.float32)
    B, n_q, Hq, d = q.shape
    L = start + n_q
    Hkv = cache["kcode"].shape[1]
    g = Hq // Hkv
    logits = np.zeros((B, n_q, Hq, L), np.float64)
    out = np.zeros((B, n_q, Hq, d), np.float64)
    vrows = {(b, h): value_rows(cache, b, h, L, value_mode, value_dtype) for b in range(B) for h in range(Hkv)}
    for t in (range(n_q) if tokens is None else tokens):
        lg, _ = decode(cache, q[:, t], U, L, kappa, value_mode, value_dtype)  # every cached token
        P = start + t
        for b in range(B):
            for a in range(Hq):
                s = lg[b, a, :P + 1]
                p = np.exp(s - s.max())
                p /= p.sum()
                logits[b, t, a, :P + 1] = s
                out[b, t, a] = p @ vrows[(b, a // g)][:P + 1]
    return logits, out
