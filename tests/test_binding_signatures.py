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


def test_keepalive_holds_every_tensor_the_struct_points_at():
    """make_paged_kv / make_ragged_kv return raw pointers in a struct; their
    keepalive must hold the pools and the device page table too, so a caller
    that keeps it cannot end up with pointers to freed memory (a page table
    freed under a live struct reads garbage page ids)."""
    import gc
    import weakref

    import numpy as np
    import torch

    def tensors():
        k = torch.zeros((4, 16, 2, 64), dtype=torch.uint8)
        return k, k.clone(), torch.tensor([0, 2, 4], dtype=torch.int32), torch.arange(4, dtype=torch.int32), \
            torch.tensor([16, 3], dtype=torch.int32)

    k, v, ip, ix, lp = tensors()
    refs = [weakref.ref(t) for t in (k, v, ip, ix, lp)]
    s, keep = fi.make_paged_kv(k, v, ip, ix, lp, kv_dtype="e4m3")
    del k, v, ip, ix, lp
    gc.collect()
    assert all(r() is not None for r in refs)
    assert s.indices == refs[3]().data_ptr() and s.k == refs[0]().data_ptr()
    del keep
    gc.collect()
    assert all(r() is None for r in refs)
    k, v, ind = torch.zeros((7, 2, 64), dtype=torch.uint8), torch.zeros((7, 2, 64), dtype=torch.uint8), \
        torch.tensor([0, 7], dtype=torch.int32)
    refs = [weakref.ref(t) for t in (k, v, ind)]
    s, keep = fi.make_ragged_kv(k, v, ind, kv_dtype="e4m3")
    del k, v, ind
    gc.collect()
    assert all(r() is not None for r in refs)
