"""Thin Python binding of libheadq (ctypes): argument marshalling only.

Every call keeps its C name: headq_calibrate, headq_calibrate_mean, headq_cache_append,
headq_decode_attn, headq_prefill_attn, headq_score_diagnostics.
PyTorch provides device memory and the current HIP stream; every step of the hot path runs in
libheadq's HIP kernels. There is no fallback: if libheadq.so is missing or fails to load, every
call raises.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path

import numpy as np

LIB_PATH = Path(__file__).resolve().parent / "libheadq.so"

HEADQ_F32, HEADQ_BF16 = 0, 1
HEADQ_V_DENSE, HEADQ_V_Q2 = 0, 1
GROUP = 32

STATUS = {
    0: "HEADQ_OK", 1: "HEADQ_ERR_NULL", 2: "HEADQ_ERR_SHAPE", 3: "HEADQ_ERR_ALIGN", 4: "HEADQ_ERR_CAPACITY",
    5: "HEADQ_ERR_WORKSPACE", 6: "HEADQ_ERR_NUMERIC", 7: "HEADQ_ERR_UNSUPPORTED", 8: "HEADQ_ERR_HIP",
}
EXPORTS = ("headq_calibrate", "headq_calibrate_mean", "headq_cache_append", "headq_decode_attn",
           "headq_prefill_attn", "headq_score_diagnostics", "headq_status_string")
DIAG_STATS = ("fisher_var", "kl", "mean_ds", "max_abs_ds", "a2", "entropy")  # HEADQ_DIAG_* order


class HeadQError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {STATUS.get(status, status)} ({status_string(status)})")


class headq_config(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("capacity", ctypes.c_int64), ("base_bits", ctypes.c_int32),
        ("group", ctypes.c_int32), ("rank", ctypes.c_int32), ("side_bits", ctypes.c_int32),
        ("key_dtype", ctypes.c_int32), ("value_dtype", ctypes.c_int32), ("value_mode", ctypes.c_int32),
        ("query_dtype", ctypes.c_int32), ("value_protect", ctypes.c_int32),
    ]


class headq_cache(ctypes.Structure):
    _fields_ = [
        ("kcode", ctypes.c_void_p), ("kmeta", ctypes.c_void_p), ("scode", ctypes.c_void_p),
        ("ssc", ctypes.c_void_p), ("v", ctypes.c_void_p), ("vcode", ctypes.c_void_p),
        ("vmeta", ctypes.c_void_p), ("U", ctypes.c_void_p), ("ktail", ctypes.c_void_p), ("vtail", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int64), ("n_pages", ctypes.c_int64),
        ("vdir", ctypes.c_void_p), ("vpidx", ctypes.c_void_p), ("vprot", ctypes.c_void_p),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree libheadq.so (built by quantized_kv_cache_headq_amd.build)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_kv_cache_headq_amd.build`")
        L = ctypes.CDLL(str(LIB_PATH))
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.headq_calibrate.argtypes = [P, P, I64, P, P]
        L.headq_calibrate_mean.argtypes = [P, P, I64, P]
        L.headq_cache_append.argtypes = [P, P, P, P, P, P, I64, I64, P, P]
        L.headq_decode_attn.argtypes = [P, P, P, I64, P, P, I32, F, P, I32, P, P, P]
        L.headq_score_diagnostics.argtypes = [P, P, P, P, P, P, P, I64, F, P, I32, P, P, P]
        L.headq_prefill_attn.argtypes = [P, P, P, I64, I64, P, I32, F, P, P]
        L.headq_status_string.argtypes = [ctypes.c_int]
        L.headq_status_string.restype = ctypes.c_char_p
        for fn in ("headq_calibrate", "headq_calibrate_mean", "headq_cache_append", "headq_decode_attn",
                   "headq_prefill_attn", "headq_score_diagnostics"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return load().headq_status_string(status).decode()
    except Exception:
        return STATUS.get(status, str(status))


def _check(status: int, call: str):
    if status != 0:
        raise HeadQError(status, call)


@dataclass
class Config:
    head_dim: int
    n_q_heads: int
    n_kv_heads: int
    batch: int
    capacity: int
    rank: int
    key_dtype: int = HEADQ_BF16
    value_dtype: int = HEADQ_BF16
    value_mode: int = HEADQ_V_DENSE
    query_dtype: int = HEADQ_BF16
    base_bits: int = 2
    group: int = GROUP
    side_bits: int = 4
    value_protect: int = 0

    def c(self) -> headq_config:
        return headq_config(self.head_dim, self.n_q_heads, self.n_kv_heads, self.batch, self.capacity,
                            self.base_bits, self.group, self.rank, self.side_bits, self.key_dtype,
                            self.value_dtype, self.value_mode, self.query_dtype, self.value_protect)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------------------------------------
# the calls

def headq_calibrate(cfg: Config, q_cal: np.ndarray):
    """Host PCA. q_cal: f32 [Hq][n_cal][d] (numpy). Returns (U f32 [Hkv][d][r], eig f64 [Hkv][r])."""
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    U = np.zeros((cfg.n_kv_heads, cfg.head_dim, cfg.rank), np.float32)
    eig = np.zeros((cfg.n_kv_heads, cfg.rank), np.float64)
    c = cfg.c()
    _check(load().headq_calibrate(ctypes.byref(c), _ptr(q), q.shape[1], _ptr(U) if cfg.rank else None, _ptr(eig)),
           "headq_calibrate")
    return U, eig


def headq_calibrate_mean(cfg: Config, q_cal: np.ndarray):
    """Host mean calibration query per KV head (the A^2 value policy's direction).
    q_cal: f32 [Hq][n_cal][d] (numpy). Returns a f32 [Hkv][d]."""
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    a = np.zeros((cfg.n_kv_heads, cfg.head_dim), np.float32)
    c = cfg.c()
    _check(load().headq_calibrate_mean(ctypes.byref(c), _ptr(q), q.shape[1], _ptr(a)), "headq_calibrate_mean")
    return a


def _strides3(t):
    if t.stride(-1) != 1:
        raise ValueError("channel stride must be 1")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def headq_cache_append(cfg: Config, cache: headq_cache, k, v=None, start: int = 0, stream=None, row_start=None):
    """Append k (and v) [B][Hkv][n_new][d] (torch device tensors) at token `start` (or at per-row
    positions row_start, a device int32 [B] tensor): whole groups are encoded, the tokens of an
    unfinished last group go to the dense tails."""
    c = cfg.c()
    ks = _strides3(k)
    vs = _strides3(v) if v is not None else None
    _check(load().headq_cache_append(ctypes.byref(c), ctypes.byref(cache), _ptr(k), ks, _ptr(v), vs, start,
                                     k.shape[2], _ptr(row_start), _stream(stream)), "headq_cache_append")


def decode_workspace_bytes(cfg: Config, n_ctx: int, n_splits: int = 0) -> int:
    c = cfg.c()
    nbytes = ctypes.c_size_t(0)
    _check(load().headq_decode_attn(ctypes.byref(c), None, None, n_ctx, None, None, 0, 1.0, None, n_splits, None,
                                    ctypes.byref(nbytes), None), "headq_decode_attn(size query)")
    return nbytes.value


def headq_decode_attn(cfg: Config, cache: headq_cache, q, n_ctx: int, out, out_dtype: int = HEADQ_F32,
                      corr_scale: float = 1.0, logits_dbg=None, n_splits: int = 0, ws=None, stream=None,
                      row_len=None):
    """One decode step: q [B][Hq][d] -> out [B][Hq][d] (torch device tensors); ws: a zero-filled device
    buffer of at least decode_workspace_bytes(cfg, n_ctx, n_splits) bytes (calls keep it reusable);
    row_len: optional device int32 [B] tokens per row (n_ctx then bounds them)."""
    c = cfg.c()
    nbytes = ctypes.c_size_t(ws.numel() * ws.element_size())
    _check(load().headq_decode_attn(ctypes.byref(c), ctypes.byref(cache), _ptr(q), n_ctx, _ptr(row_len), _ptr(out),
                                    out_dtype,
                                    float(corr_scale), _ptr(logits_dbg), n_splits, _ptr(ws), ctypes.byref(nbytes),
                                    _stream(stream)), "headq_decode_attn")


def headq_prefill_attn(cfg: Config, cache: headq_cache, q, start: int, out, out_dtype: int = HEADQ_F32,
                       corr_scale: float = 1.0, logits_dbg=None, stream=None):
    """Chunked-prefill attention: q [B][n_q][Hq][d] (torch device tensor, query dtype), query token
    t at position start + t attending cached tokens 0 .. start + t; out [B][n_q][Hq][d];
    logits_dbg: optional f32 [B][n_q][Hq][start + n_q]."""
    c = cfg.c()
    _check(load().headq_prefill_attn(ctypes.byref(c), ctypes.byref(cache), _ptr(q), start, q.shape[1], _ptr(out),
                                     out_dtype, float(corr_scale), _ptr(logits_dbg), _stream(stream)),
           "headq_prefill_attn")


def diagnostics_workspace_bytes(cfg: Config, n_ctx: int, n_splits: int = 0) -> int:
    c = cfg.c()
    nbytes = ctypes.c_size_t(0)
    _check(load().headq_score_diagnostics(ctypes.byref(c), None, None, None, None, None, None, n_ctx, 1.0, None,
                                          n_splits, None, ctypes.byref(nbytes), None),
           "headq_score_diagnostics(size query)")
    return nbytes.value


def headq_score_diagnostics(cfg: Config, cache: headq_cache, q, k_ref, v_ref, n_ctx: int, stats,
                            corr_scale: float = 1.0, n_splits: int = 0, ws=None, stream=None):
    """Score-space diagnostics of the cache against reference keys k_ref (and values v_ref, or
    None) [B][Hkv][>= n_ctx][d] (torch device tensors): stats, a device f64 [B][Hq][6] tensor, gets
    DIAG_STATS per (b, query head). ws: device buffer of diagnostics_workspace_bytes(...) bytes."""
    c = cfg.c()
    nbytes = ctypes.c_size_t(ws.numel() * ws.element_size())
    vs = _strides3(v_ref) if v_ref is not None else None
    _check(load().headq_score_diagnostics(ctypes.byref(c), ctypes.byref(cache), _ptr(q), _ptr(k_ref),
                                          _strides3(k_ref), _ptr(v_ref), vs, n_ctx, float(corr_scale), _ptr(stats),
                                          n_splits, _ptr(ws), ctypes.byref(nbytes), _stream(stream)),
           "headq_score_diagnostics")


# ------------------------------------------------------------------------------------------------
# device buffers of one layer's cache (torch for memory only)

class DeviceCache:
    """Caller-owned device buffers of one layer in libheadq's cache format."""

    def __init__(self, cfg: Config, device="cuda"):
        import torch
        self.cfg = cfg
        B, H, cap, d, r = cfg.batch, cfg.n_kv_heads, cfg.capacity, cfg.head_dim, cfg.rank
        u8, i16 = torch.uint8, torch.int16
        self.kcode = torch.zeros((B, H, cap, d // 4 if cfg.base_bits == 2 else d // 2), dtype=u8, device=device)
        self.kmeta = torch.zeros((B, H, cap // GROUP, 2, d), dtype=i16, device=device)
        self.scode = torch.zeros((B, H, cap, max(r // 2, 1)), dtype=u8, device=device) if r else None
        self.ssc = torch.zeros((B, H, cap), dtype=i16, device=device) if r else None
        self.v = self.vcode = self.vmeta = None
        if cfg.value_mode == HEADQ_V_DENSE:
            vdt = torch.float32 if cfg.value_dtype == HEADQ_F32 else torch.bfloat16
            self.v = torch.zeros((B, H, cap // GROUP, d, GROUP), dtype=vdt, device=device)
        else:
            self.vcode = torch.zeros((B, H, cap // GROUP, d * 8), dtype=u8, device=device)
            self.vmeta = torch.zeros((B, H, cap // GROUP, 2, d // GROUP, GROUP), dtype=i16, device=device)
        kdt = torch.float32 if cfg.key_dtype == HEADQ_F32 else torch.bfloat16
        vdt = torch.float32 if cfg.value_dtype == HEADQ_F32 else torch.bfloat16
        self.ktail = torch.zeros((B, H, GROUP, d), dtype=kdt, device=device)
        self.vtail = torch.zeros((B, H, GROUP, d), dtype=vdt, device=device)
        self.U = None
        self.vdir = None
        Pv = cfg.value_protect
        self.vpidx = torch.zeros((B, H, cap // GROUP), dtype=torch.int32, device=device) if Pv else None
        self.vprot = torch.zeros((B, H, cap // GROUP, Pv, d), dtype=i16, device=device) if Pv else None

    def set_basis(self, U):
        import torch
        self.U = torch.as_tensor(np.ascontiguousarray(U, np.float32)).to(self.kcode.device)

    def set_direction(self, a):
        """The A^2 value policy's direction (headq_calibrate_mean's output), f32 [Hkv][d]."""
        import torch
        self.vdir = torch.as_tensor(np.ascontiguousarray(a, np.float32)).to(self.kcode.device)

    def c(self) -> headq_cache:
        return headq_cache(_ptr(self.kcode), _ptr(self.kmeta), _ptr(self.scode), _ptr(self.ssc), _ptr(self.v),
                           _ptr(self.vcode), _ptr(self.vmeta), _ptr(self.U), _ptr(self.ktail), _ptr(self.vtail),
                           None, 0, 0, _ptr(self.vdir), _ptr(self.vpidx), _ptr(self.vprot))

    def append(self, k, v=None, start: int = 0, stream=None, row_start=None):
        headq_cache_append(self.cfg, self.c(), k, v, start, stream, row_start)

    def decode(self, q, n_ctx: int, out=None, out_dtype: int = HEADQ_F32, corr_scale: float = 1.0, logits_dbg=None,
               n_splits: int = 0, ws=None, stream=None, row_len=None):
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32 if out_dtype == HEADQ_F32 else torch.bfloat16,
                              device=q.device)
        if ws is None:
            nb = decode_workspace_bytes(self.cfg, n_ctx, n_splits)
            ws = torch.zeros((nb + 3) // 4, dtype=torch.float32, device=q.device)
        headq_decode_attn(self.cfg, self.c(), q, n_ctx, out, out_dtype, corr_scale, logits_dbg, n_splits, ws, stream,
                          row_len)
        return out

    def prefill(self, q, start: int, out=None, out_dtype: int = HEADQ_F32, corr_scale: float = 1.0,
                logits_dbg=None, stream=None):
        import torch
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32 if out_dtype == HEADQ_F32 else torch.bfloat16,
                              device=q.device)
        headq_prefill_attn(self.cfg, self.c(), q, start, out, out_dtype, corr_scale, logits_dbg, stream)
        return out

    def score_diagnostics(self, q, k_ref, v_ref, n_ctx: int, corr_scale: float = 1.0, n_splits: int = 0, ws=None,
                          stream=None):
        """f64 [B][Hq][6] statistics (DIAG_STATS order) of this cache against k_ref / v_ref."""
        import torch
        if ws is None:
            nb = diagnostics_workspace_bytes(self.cfg, n_ctx, n_splits)
            ws = torch.empty((nb + 7) // 8, dtype=torch.float64, device=q.device)
        stats = torch.empty((self.cfg.batch, self.cfg.n_q_heads, len(DIAG_STATS)), dtype=torch.float64,
                            device=q.device)
        headq_score_diagnostics(self.cfg, self.c(), q, k_ref, v_ref, n_ctx, stats, corr_scale, n_splits, ws, stream)
        return stats

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.kcode, self.kmeta, self.scode, self.ssc, self.v,
                                                           self.vcode, self.vmeta, self.ktail, self.vtail,
                                                           self.vpidx, self.vprot)
                   if t is not None)


class PagedDeviceCache(DeviceCache):
    """A paged cache: every packed array is a pool of n_pages pages (one page = one 32-token group
    of all KV heads), and group g of batch row b lives in page block_table[b][g]. The tails stay per
    row. block_table is a device int32 [B][max_pages] tensor the caller fills (and may change
    between calls); cfg.capacity is the per-row logical capacity, at most 32 * max_pages."""

    def __init__(self, cfg: Config, n_pages: int, max_pages: int, device="cuda"):
        import torch
        if cfg.capacity > GROUP * max_pages:
            raise ValueError("capacity exceeds 32 * max_pages")
        self.cfg = cfg
        self.n_pages, self.max_pages = n_pages, max_pages
        H, d, r, P = cfg.n_kv_heads, cfg.head_dim, cfg.rank, n_pages
        u8, i16 = torch.uint8, torch.int16
        self.kcode = torch.zeros((P, H, GROUP, d // 4 if cfg.base_bits == 2 else d // 2), dtype=u8, device=device)
        self.kmeta = torch.zeros((P, H, 2, d), dtype=i16, device=device)
        self.scode = torch.zeros((P, H, GROUP, max(r // 2, 1)), dtype=u8, device=device) if r else None
        self.ssc = torch.zeros((P, H, GROUP), dtype=i16, device=device) if r else None
        self.v = self.vcode = self.vmeta = None
        if cfg.value_mode == HEADQ_V_DENSE:
            vdt = torch.float32 if cfg.value_dtype == HEADQ_F32 else torch.bfloat16
            self.v = torch.zeros((P, H, d, GROUP), dtype=vdt, device=device)
        else:
            self.vcode = torch.zeros((P, H, d * 8), dtype=u8, device=device)
            self.vmeta = torch.zeros((P, H, 2, d // GROUP, GROUP), dtype=i16, device=device)
        kdt = torch.float32 if cfg.key_dtype == HEADQ_F32 else torch.bfloat16
        vdt = torch.float32 if cfg.value_dtype == HEADQ_F32 else torch.bfloat16
        self.ktail = torch.zeros((cfg.batch, H, GROUP, d), dtype=kdt, device=device)
        self.vtail = torch.zeros((cfg.batch, H, GROUP, d), dtype=vdt, device=device)
        self.block_table = torch.zeros((cfg.batch, max_pages), dtype=torch.int32, device=device)
        self.U = None
        self.vdir = None
        Pv = cfg.value_protect
        self.vpidx = torch.zeros((P, H), dtype=torch.int32, device=device) if Pv else None
        self.vprot = torch.zeros((P, H, Pv, d), dtype=i16, device=device) if Pv else None

    def c(self) -> headq_cache:
        return headq_cache(_ptr(self.kcode), _ptr(self.kmeta), _ptr(self.scode), _ptr(self.ssc), _ptr(self.v),
                           _ptr(self.vcode), _ptr(self.vmeta), _ptr(self.U), _ptr(self.ktail), _ptr(self.vtail),
                           _ptr(self.block_table), self.max_pages, self.n_pages, _ptr(self.vdir), _ptr(self.vpidx),
                           _ptr(self.vprot))
