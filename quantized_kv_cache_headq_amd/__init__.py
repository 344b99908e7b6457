"""libheadq — the HeadQ key-side KV-cache hot path for AMD Instinct MI355X (gfx950).

The compute lives in libheadq.so (hand-written HIP kernels behind a C ABI declared in
include/headq.h); this package only marshals arguments to it.
"""
from .binding import (DIAG_STATS, EXPORTS, HEADQ_BF16, HEADQ_F32, HEADQ_V_DENSE, HEADQ_V_Q2, Config, DeviceCache,
                      HeadQError, PagedDeviceCache, decode_workspace_bytes, diagnostics_workspace_bytes,
                      headq_cache_append, headq_calibrate, headq_calibrate_mean, headq_decode_attn, headq_prefill_attn,
                      headq_score_diagnostics, load)

__all__ = ["DIAG_STATS", "EXPORTS", "HEADQ_BF16", "HEADQ_F32", "HEADQ_V_DENSE", "HEADQ_V_Q2", "Config", "DeviceCache",
           "HeadQError", "PagedDeviceCache", "decode_workspace_bytes", "diagnostics_workspace_bytes",
           "headq_cache_append", "headq_calibrate", "headq_calibrate_mean", "headq_decode_attn", "headq_prefill_attn",
           "headq_score_diagnostics", "load"]
