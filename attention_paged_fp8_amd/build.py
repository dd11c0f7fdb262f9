"""Build libfi.so (the HIP library behind include/fi.h) in-tree for gfx950.

    python -m attention_paged_fp8_amd.build             # or build() from Python
    python -m attention_paged_fp8_amd.build --sanitize  # host front end under ASan + UBSan

--sanitize builds a second library, attention_paged_fp8_amd/_sanitize/libfi.so,
whose host front end (fi_api.cpp: argument checks, planning, launches) is
compiled and linked with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only; the kernels are built as usual).  sanitize_check.py runs the
CPU tests of the C ABI against it.

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

SOURCES = ["fi_api.cpp", "fi_decode.hip", "fi_prefill.hip", "fi_pod.hip"]
HEADERS = ["fi_internal.h", "fi_device.hpp", "fi_decode_body.hpp", "fi_prefill_body.hpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Host-only sanitizer flags of the --sanitize build (applied to fi_api.cpp and the link).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_LIB = os.path.join(HERE, "_sanitize", "libfi.so")
# Per-source flags.  The prefill kernel zeroes every out-of-range or poisoned
# element before it reaches arithmetic, so it produces no NaN; without IEEE-mode
# NaN quieting its max reductions take one instruction per element instead of
# three.  (The decode kernel gains nothing from this and spills with it.)  The
# fused kernel runs the prefill body, and its decode body tolerates the flags.
PER_SOURCE = {"fi_prefill.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
              "fi_pod.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str, extra: list[str], csrc: str = CSRC, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *PER_SOURCE.get(src, []), f"-I{csrc}", *extra, "-c", os.path.join(csrc, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB, csrc: str = CSRC,
          sanitize: bool = False) -> str:
    """Compile every source and link the library (default libfi.so in the
    package; `out`, `csrc` and `extra` build a variant elsewhere; `sanitize`
    builds the ASan + UBSan host front end into _sanitize/libfi.so); returns
    its path."""
    if sanitize and out == LIB:
        out = SANITIZE_LIB
    build_dir = BUILD if out == LIB else os.path.splitext(out)[0] + "_build"
    os.makedirs(build_dir, exist_ok=True)
    extra = list(extra or [])
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    per = (lambda src: extra + SANITIZE) if sanitize else (lambda src: extra)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, per(s) if s == "fi_api.cpp" else extra, csrc, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *(SANITIZE if sanitize else []), *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    san = "--sanitize" in args
    build(verbose=True, extra=[a for a in args if a != "--sanitize"], sanitize=san)
