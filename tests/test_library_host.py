"""libheadq host-side tests (CPU only): exports, headq_calibrate, argument validation.

Argument checks run before any HIP call, so every rejected call here touches no GPU.
"""
import ctypes
import re
import subprocess
import sys

import numpy as np
import pytest

import quantized_kv_cache_headq_amd as hq
from quantized_kv_cache_headq_amd import binding as bd
from oracle import oracle as orc
from workloads import synth

from .conftest import ROOT


def _header_functions():
    text = open(f"{ROOT}/include/headq.h").read()
    return sorted(set(re.findall(r"^(?:headq_status|const char\*)\s+(headq_\w+)\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    declared = _header_functions()
    assert declared == sorted(["headq_calibrate", "headq_calibrate_mean", "headq_cache_append", "headq_decode_attn",
                               "headq_prefill_attn", "headq_score_diagnostics", "headq_status_string"])
    out = subprocess.run(["nm", "-D", "--defined-only", str(bd.LIB_PATH)], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (headq_\w+)", out))
    assert set(declared) <= exported
    lib = hq.load()
    for name in declared:
        assert getattr(lib, name) is not None


def test_status_strings():
    for code in range(9):
        s = bd.status_string(code)
        assert isinstance(s, str) and s


def _cfg(**kw):
    base = dict(head_dim=64, n_q_heads=4, n_kv_heads=2, batch=1, capacity=128, rank=8, key_dtype=bd.HEADQ_F32,
                value_dtype=bd.HEADQ_F32, query_dtype=bd.HEADQ_F32)
    base.update(kw)
    return bd.Config(**base)


# ------------------------------------------------------------------------------------------------
# headq_calibrate (host PCA) against the oracle's Jacobi PCA and numpy.linalg.eigh

@pytest.mark.parametrize("wname", ["tiny", "qwen7b_decode"])
def test_calibrate_matches_oracle_and_eigh(wname):
    w = synth.WORKLOADS[wname]
    if w.n_q_heads > 8:
        w = synth.scaled(w, n_q_heads=w.n_kv_heads * w.gqa)
    qc = synth.calibration_queries(w, n_cal=256)
    cfg = _cfg(head_dim=w.head_dim, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, rank=w.rank)
    U, eig = hq.headq_calibrate(cfg, qc)
    Uo, eigo = orc.calibrate(qc, w.n_kv_heads, w.rank)
    g = w.gqa
    for h in range(w.n_kv_heads):
        X = qc[h * g:(h + 1) * g].reshape(-1, w.head_dim).astype(np.float64)
        lam = np.linalg.eigvalsh(X.T @ X / X.shape[0])[::-1]
        assert np.allclose(eig[h], lam[:w.rank], rtol=1e-9)
        assert np.allclose(eig[h], eigo[h], rtol=1e-9)
        gaps = lam[:w.rank] - lam[1:w.rank + 1]
        if np.all(gaps > 1e-6 * lam[0]):
            # same sign rule on both sides: columns agree, not only the subspace
            assert np.allclose(U[h], Uo[h], atol=2e-5)
        P = U[h].astype(np.float64) @ U[h].T
        Po = Uo[h].astype(np.float64) @ Uo[h].T
        assert np.linalg.norm(P - Po) < 1e-5
        assert np.allclose(U[h].T.astype(np.float64) @ U[h], np.eye(w.rank), atol=1e-6)


def test_calibrate_rejects_bad_input():
    cfg = _cfg()
    q = np.zeros((4, 16, 64), np.float32)
    q[0, 0, 0] = np.nan
    with pytest.raises(hq.HeadQError) as e:
        hq.headq_calibrate(cfg, q)
    assert e.value.status == 6
    with pytest.raises(hq.HeadQError) as e:
        hq.headq_calibrate(_cfg(rank=12), np.ones((4, 16, 64), np.float32))
    assert e.value.status == 7
    with pytest.raises(hq.HeadQError) as e:
        hq.headq_calibrate(_cfg(n_q_heads=3), np.ones((3, 16, 64), np.float32))
    assert e.value.status == 2


# ------------------------------------------------------------------------------------------------
# argument validation of the GPU calls (all rejected before any HIP call)

class _FakeDev:
    """Stands in for a device tensor: only a pointer and strides are read before validation fails."""

    def __init__(self, addr, shape, strides):
        self.addr, self.shape, self._strides = addr, shape, strides

    def data_ptr(self):
        return self.addr

    def stride(self, i=None):
        return self._strides if i is None else self._strides[i]


def _append_status(cfg, cache, k, v=None, start=0, n_new=None, row_start=None):
    lib = hq.load()
    c = cfg.c()
    ks = (ctypes.c_int64 * 3)(*k._strides[:3]) if k is not None else None
    vs = (ctypes.c_int64 * 3)(*v._strides[:3]) if v is not None else None
    n = k.shape[2] if n_new is None else n_new
    return lib.headq_cache_append(ctypes.byref(c), ctypes.byref(cache) if cache is not None else None,
                                  k.addr if k is not None else None, ks, v.addr if v is not None else None, vs,
                                  start, n, row_start, None)


def _fake_cache(cfg):
    base = 0x10000000
    return bd.headq_cache(base, base + 0x1000, base + 0x2000, base + 0x3000, base + 0x4000, base + 0x5000,
                          base + 0x6000, base + 0x7000)


def _fake_keys(cfg, n=64, align=0):
    d = cfg.head_dim
    return _FakeDev(0x20000000 + align, (cfg.batch, cfg.n_kv_heads, n, d),
                    (cfg.n_kv_heads * n * d, n * d, d, 1))


def test_append_validation_statuses():
    cfg = _cfg()
    cache = _fake_cache(cfg)
    k = _fake_keys(cfg)
    assert _append_status(cfg, None, k) == 1                                  # NULL cache
    assert _append_status(_cfg(head_dim=96), cache, k) == 7                   # unsupported d
    assert _append_status(_cfg(rank=12), cache, k) == 7                       # unsupported rank
    assert _append_status(_cfg(n_q_heads=6, n_kv_heads=4), cache, k) == 2     # Hq % Hkv
    assert _append_status(_cfg(n_q_heads=34, n_kv_heads=2), cache, k) == 7    # g > 16
    assert _append_status(_cfg(capacity=100), cache, k) == 3                  # capacity % 32
    assert _append_status(cfg, cache, k, start=16) == 1                       # inside a group, no tails
    assert _append_status(cfg, cache, k, n_new=48) == 1                       # ends inside a group, no tails
    assert _append_status(cfg, cache, k, row_start=0x60000000) == 1           # per-row positions need tails
    assert _append_status(cfg, cache, k, start=96) == 4                       # start + n > cap
    assert _append_status(cfg, cache, _fake_keys(cfg, align=4)) == 3          # misaligned keys
    bad = bd.headq_cache(0x10000004, 0x10001000, 0x10002000, 0x10003000, 0x10004000, 0, 0, 0x10007000)
    assert _append_status(cfg, bad, k) == 3                                   # misaligned cache
    nos = bd.headq_cache(0x10000000, 0x10001000, 0, 0, 0x10004000, 0, 0, 0)
    assert _append_status(cfg, nos, k) == 1                                   # rank > 0 without side buffers
    assert _append_status(_cfg(rank=0), nos, k, n_new=0) == 0                 # n_new == 0 is a no-op
    q2 = _cfg(value_mode=bd.HEADQ_V_Q2)
    assert _append_status(q2, bd.headq_cache(0x10000000, 0x10001000, 0x10002000, 0x10003000, 0, 0, 0,
                                               0x10007000), k) == 1          # 2-bit values need vcode/vmeta


def _paged(cfg, max_pages, n_pages, table=0x70000000):
    c = _fake_cache(cfg)
    c.ktail, c.vtail = 0x11000000, 0x12000000
    c.block_table, c.max_pages, c.n_pages = table, max_pages, n_pages
    return c


def test_paged_cache_validation_statuses():
    cfg = _cfg()  # capacity 128 = 4 groups per row
    k = _fake_keys(cfg)
    assert _append_status(cfg, _paged(cfg, 0, 8), k) == 2                    # no table columns
    assert _append_status(cfg, _paged(cfg, 4, 0), k) == 2                    # empty pools
    assert _append_status(cfg, _paged(cfg, 3, 8), k) == 2                    # capacity > 32 * max_pages
    assert _append_status(cfg, _paged(cfg, 4, 8, table=0x70000002), k) == 3  # misaligned table
    assert _decode_status(cfg, cache=_paged(cfg, 3, 8))[0] == 2
    assert _decode_status(cfg, cache=_paged(cfg, 4, 8, table=0x70000002))[0] == 3


def _decode_status(cfg, cache=None, q=0x30000000, n_ctx=64, out=0x40000000, ws=0x50000000, nbytes=1 << 20,
                   n_splits=0, out_dtype=0, row_len=None):
    lib = hq.load()
    c = cfg.c()
    nb = ctypes.c_size_t(nbytes)
    cache = _fake_cache(cfg) if cache is None else cache
    st = lib.headq_decode_attn(ctypes.byref(c), ctypes.byref(cache), q, n_ctx, row_len, out, out_dtype, 1.0, None,
                               n_splits, ws, ctypes.byref(nb), None)
    return st, nb.value


def test_decode_workspace_query_and_validation():
    cfg = _cfg(batch=2)
    st, nb = _decode_status(cfg, ws=None, nbytes=0)
    assert st == 0 and nb > 0
    st1, nb1 = _decode_status(cfg, ws=None, nbytes=0, n_splits=1)
    assert st1 == 0 and nb1 == 256 + 2 * 4 * 1 * (64 + 2) * 4  # counters (padded), then partials
    assert _decode_status(cfg, nbytes=nb1 - 4, n_splits=1)[0] == 5           # workspace too small
    assert _decode_status(cfg, n_ctx=48)[0] == 1                              # n_ctx % 32 without tails
    assert _decode_status(cfg, n_ctx=160)[0] == 4                             # n_ctx > capacity
    assert _decode_status(cfg, n_ctx=0)[0] == 2
    assert _decode_status(cfg, n_splits=3)[0] == 2                            # more splits than groups
    assert _decode_status(cfg, n_ctx=48, n_splits=3)[0] == 2                  # 1 whole group + the tail
    assert _decode_status(cfg, row_len=0x60000000)[0] == 1                    # per-row lengths need tails
    assert _decode_status(cfg, q=0x30000002)[0] == 3                          # misaligned query
    assert _decode_status(cfg, out_dtype=5)[0] == 7
    assert _decode_status(cfg, q=None)[0] == 1
    assert hq.decode_workspace_bytes(cfg, 64, 2) == 256 + 2 * 4 * 2 * 66 * 4


def _diag_status(cfg, cache=None, q=0x30000000, k=None, v=None, n_ctx=64, stats=0x40000000, ws=0x50000000,
                 nbytes=1 << 20, n_splits=0):
    lib = hq.load()
    c = cfg.c()
    cache = _fake_cache(cfg) if cache is None else cache
    k = _fake_keys(cfg) if k is None else k
    nb = ctypes.c_size_t(nbytes)
    ks = (ctypes.c_int64 * 3)(*k._strides[:3])
    vs = (ctypes.c_int64 * 3)(*v._strides[:3]) if v is not None else None
    st = lib.headq_score_diagnostics(ctypes.byref(c), ctypes.byref(cache), q, k.addr, ks,
                                     v.addr if v is not None else None, vs, n_ctx, 1.0, stats, n_splits, ws,
                                     ctypes.byref(nb), None)
    return st, nb.value


def test_score_diagnostics_workspace_query_and_validation():
    cfg = _cfg()
    st, nb = _diag_status(cfg, ws=None, nbytes=0)
    assert st == 0 and nb > 0
    st2, nb2 = _diag_status(cfg, ws=None, nbytes=0, n_ctx=128)
    assert st2 == 0 and nb2 > nb                                              # per-token value errors
    assert _diag_status(cfg, nbytes=nb - 8)[0] == 5                          # workspace too small
    assert _diag_status(cfg, n_ctx=48)[0] == 1                               # n_ctx % 32 without tails
    assert _diag_status(cfg, n_ctx=160)[0] == 4                              # n_ctx > capacity
    assert _diag_status(cfg, n_ctx=0)[0] == 2
    assert _diag_status(cfg, n_splits=2)[0] == 2                             # more splits than 64-token chunks
    assert _diag_status(cfg, q=0x30000004)[0] == 3                           # misaligned query
    assert _diag_status(cfg, stats=0x40000008)[0] == 3                       # misaligned statistics
    assert _diag_status(cfg, k=_fake_keys(cfg, align=4))[0] == 3             # misaligned keys
    assert _diag_status(cfg, stats=None)[0] == 1
    assert _diag_status(cfg, cache=_paged(cfg, 3, 8))[0] == 2                # paged: capacity > 32 * max_pages


def _prefill_status(cfg, cache=None, q=0x30000000, start=32, n_q=64, out=0x40000000, out_dtype=0, logits=None):
    lib = hq.load()
    c = cfg.c()
    cache = _fake_cache(cfg) if cache is None else cache
    return lib.headq_prefill_attn(ctypes.byref(c), ctypes.byref(cache), q, start, n_q, out, out_dtype, 1.0, logits,
                                  None)


def test_prefill_validation_statuses():
    cfg = _cfg(value_dtype=bd.HEADQ_BF16)                                # capacity 128
    assert _prefill_status(cfg, n_q=0) == 2
    assert _prefill_status(cfg, start=-1) == 2
    assert _prefill_status(cfg, start=100, n_q=29) == 4                  # past the capacity
    assert _prefill_status(cfg, start=3) == 1                            # ends inside a group, no tails
    assert _prefill_status(_cfg(), start=32) == 7                        # dense f32 values: not a matrix-core format
    assert _prefill_status(cfg, q=0x30000004) == 3
    assert _prefill_status(cfg, logits=0x50000008) == 3
    assert _prefill_status(cfg, out_dtype=3) == 7
    assert _prefill_status(cfg, q=None) == 1
    assert _prefill_status(cfg, cache=_paged(cfg, 3, 8)) == 2            # paged: capacity > 32 * max_pages


def test_calibrate_mean_matches_the_oracle_bit_for_bit():
    """The policy's direction: the library's host mean and the oracle's take the same f64 sums in the
    same order, so the f32 results agree exactly."""
    w = synth.scaled(synth.WORKLOADS["qwen7b_decode"], n_q_heads=14, n_kv_heads=2)
    q = synth.calibration_queries(w, n_cal=96)
    cfg = hq.Config(head_dim=w.head_dim, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, batch=1, capacity=32,
                    rank=w.rank)
    a = hq.headq_calibrate_mean(cfg, q)
    assert np.array_equal(a.view(np.uint32), orc.mean_query(q, w.n_kv_heads).view(np.uint32))


def test_value_policy_settings_are_validated():
    w = synth.scaled(synth.WORKLOADS["qwen14b_fullkv"], n_q_heads=10, n_kv_heads=2)
    base = dict(head_dim=w.head_dim, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, batch=1, capacity=64,
                rank=w.rank, value_mode=bd.HEADQ_V_Q2)
    q = np.zeros((1, 10, 128), np.float32)
    for bad in (dict(value_protect=3), dict(value_protect=-1), dict(value_protect=1, value_mode=bd.HEADQ_V_DENSE),
                dict(value_protect=1, base_bits=4)):
        cfg = hq.Config(**{**base, **bad})
        with pytest.raises(hq.HeadQError, match="UNSUPPORTED"):
            hq.decode_workspace_bytes(cfg, 64)
    # the policy needs its direction, indices and corrections (checked before any GPU call)
    cfg = hq.Config(**base, value_protect=2)
    buf = np.zeros(64, np.uint64)  # 16-byte aligned stand-in address for every other buffer
    addr = buf.ctypes.data
    cache = bd.headq_cache(addr, addr, addr, addr, None, addr, addr, addr, addr, addr, None, 0, 0, None, addr, addr)
    lib = hq.load()
    st = lib.headq_cache_append(ctypes.byref(cfg.c()), ctypes.byref(cache), 16, (ctypes.c_int64 * 3)(1, 1, 128),
                                None, None, 0, 32, None, None)
    assert bd.STATUS[st] == "HEADQ_ERR_NULL"


def test_missing_library_fails_loudly():
    """Without the built library every call raises: there is no CPU or torch fallback."""
    code = ("import pathlib, numpy as np\n"
            "import quantized_kv_cache_headq_amd as hq\n"
            "import quantized_kv_cache_headq_amd.binding as bd\n"
            "bd.LIB_PATH = pathlib.Path('/nonexistent/libheadq.so')\n"
            "cfg = hq.Config(128, 28, 4, 1, 64, 16)\n"
            "try:\n"
            "    hq.headq_calibrate(cfg, np.zeros((28, 8, 128), np.float32))\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "is missing" in r.stdout
