"""The ctypes binding declares each C entry point with the parameters its
prototype in include/fi.h has: same count, and each pointer, 32-bit integer
(or fi_dtype enum), 64-bit integer, float or size_t in the same position (CPU
only; no call is made)."""
import ctypes
import os
import re

import pytest

from attention_paged_fp8_amd import fi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fi.h")


def _prototypes():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"^(?:fi_status|size_t|const char\*)\s+(fi_\w+)\s*\(([^)]*)\)\s*;", src, re.M):
        params = [p.strip() for p in m.group(2).replace("\n", " ").split(",") if p.strip() and p.strip() != "void"]
        out[m.group(1)] = params
    return out


def _kind(c_param: str) -> str:
    t = c_param.rsplit(" ", 1)[0] if not c_param.endswith("*") else c_param
    if "*" in c_param:
        return "ptr"
    if "fi_dtype" in t:  # a C enum: int-sized in this ABI
        return "i32"
    if "int64_t" in t:
        return "i64"
    if "int32_t" in t:
        return "i32"
    if "size_t" in t:
        return "size"
    if "float" in t:
        return "f32"
    raise AssertionError(c_param)


def _ctype_kind(t) -> str:
    if t is ctypes.c_void_p or (isinstance(t, type) and issubclass(t, ctypes._Pointer)):
        return "ptr"
    if t in (ctypes.c_int, ctypes.c_int32):  # the same type where int is 32 bits
        return "i32"
    if t is ctypes.c_int64:
        return "i64"
    if t is ctypes.c_int32:
        return "i32"
    if t is ctypes.c_size_t:
        return "size"
    if t is ctypes.c_float:
        return "f32"
    raise AssertionError(t)


PROTOS = _prototypes()


def test_every_export_has_a_prototype():
    assert sorted(PROTOS) == sorted(fi.EXPORTS)


@pytest.mark.parametrize("name", sorted(PROTOS))
def test_binding_matches_prototype(name):
    L = fi.lib()
    fn = getattr(L, name)
    want = [_kind(p) for p in PROTOS[name]]
    got = [_ctype_kind(t) for t in (fn.argtypes or [])]
    assert got == want, f"{name}: binding {got} against header {want}"
