"""Run the C ABI's CPU tests against the ASan + UBSan build of the host front end.

    python -m attention_paged_fp8_amd.sanitize_check

Builds attention_paged_fp8_amd/_sanitize/libfi.so (build(sanitize=True): the
argument checks, planning and launch code of fi_api.cpp compiled and linked
with -fsanitize=address and -fsanitize=undefined, host code only, undefined
behaviour fatal), then runs tests/test_abi.py and
tests/test_binding_signatures.py in a child Python with the AddressSanitizer
runtime preloaded and FI_LIB_PATH naming that library.  For a host without a
GPU: every refusal path, the host page-table checks and the planners run; no
kernel is launched.  Exits with pytest's status.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from attention_paged_fp8_amd.build import ROOT, SANITIZE_LIB, build


def asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("the clang AddressSanitizer runtime (libclang_rt.asan-x86_64.so) was not found under "
                           "/opt/rocm/llvm")
    return hits[-1]


def main() -> int:
    build(verbose=True, sanitize=True)
    env = dict(os.environ)
    env["FI_LIB_PATH"] = SANITIZE_LIB
    env["LD_PRELOAD"] = asan_runtime()
    # the interpreter itself is not instrumented: leaks at exit are Python's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py"),
           os.path.join(ROOT, "tests", "test_binding_signatures.py")]
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main())
