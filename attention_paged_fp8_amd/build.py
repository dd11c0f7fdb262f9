"""Build libfi.so (the HIP library behind include/fi.h) in-tree for gfx950.

    python -m attention_paged_fp8_amd.build        # or build() from Python

Every translation unit is compiled by hipcc for --offload-arch=gfx950 in
parallel into _build/, then linked into attention_paged_fp8_amd/libfi.so.
Packed-fp32 instruction selection is disabled
(-target-feature -packed-fp32-ops): hipcc may otherwise fuse pairs of fp32
operations into v_pk_*_f32 forms that this library does not rely on.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["fi_api.cpp", "fi_decode.hip", "fi_prefill.hip"]
HEADERS = ["fi_internal.h", "fi_device.hpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Per-source flags.  The prefill kernel zeroes every out-of-range or poisoned
# element before it reaches arithmetic, so it produces no NaN; without IEEE-mode
# NaN quieting its max reductions take one instruction per element instead of
# three.  (The decode kernel gains nothing from this and spills with it.)
PER_SOURCE = {"fi_prefill.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str, extra: list[str], csrc: str = CSRC, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *PER_SOURCE.get(src, []), f"-I{csrc}", *extra, "-c", os.path.join(csrc, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB, csrc: str = CSRC) -> str:
    """Compile every source and link the library (default libfi.so in the
    package; `out`, `csrc` and `extra` build a variant elsewhere); returns its path."""
    build_dir = BUILD if out == LIB else os.path.splitext(out)[0] + "_build"
    os.makedirs(build_dir, exist_ok=True)
    extra = list(extra or [])
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, csrc, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
