"""Build libheadq.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m quantized_kv_cache_headq_amd.build   (or call build_library()).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OUT = PKG / "libheadq.so"
BUILD_DIR = PKG / "_build"

SOURCES = ["headq_api.cpp", "calibrate.cpp", "append.hip", "decode.hip", "decode_mfma.hip", "diagnostics.hip",
           "prefill_mfma.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # packed-fp32 instructions stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math", "-Wall", "-Wno-unused-function",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> Path:
    obj = BUILD_DIR / (Path(src).stem + ".o")
    cmd = [_hipcc(), *COMMON, "-c", str(CSRC / src), "-o", str(obj)]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build_library(verbose: bool = False) -> Path:
    """Compile every source for gfx950 and link libheadq.so (always rebuilds)."""
    BUILD_DIR.mkdir(exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
