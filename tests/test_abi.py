"""C-ABI tests that need no GPU (CPU only).

* libfi.so loads and exports every function include/fi.h declares.
* Each refusal returns its status and a sentence naming the call, the
  argument and the dtype(s), before any HIP call: the refusal set of "fp8 KV
  cache in the in-tree prefill kernel" (AMD-Ecosystem/flashinfer PR #368,
  Refusals and Test plan: fp8 query, integer KV, float32, mismatched k/v,
  prefill 2-byte KV that differs from q) and of "Enable Hopper FA3 FP8
  attention in decode.py" (flashinfer PR #2148, Walkthrough: fp8 output).

Device pointers here are NULL (or, for checks that come after the NULL check,
fake addresses), so these tests never reach a kernel; they are skipped where a
GPU is visible, and the same refusals are exercised on the GPU with real
tensors by test_gpu_decode.py.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

from attention_paged_fp8_amd import fi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fi.h")

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer refusal checks run only without a GPU")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fi.LIB_PATH):
        from attention_paged_fp8_amd.build import build
        build()
    return fi.lib()


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:fi_status|size_t|const char\*)\s+(fi_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) == 14, names
    assert sorted(fi.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fi.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), f"{n} not exported as a text symbol"


def test_workspace_bound(L):
    assert fi.fi_decode_workspace_bytes(0, 32, 128, 4096) == 0
    # B * H_qo * (ceil(max_kv / 64) + 1) pieces * (D + 1) floats, plus B * H_qo piece counts
    assert fi.fi_decode_workspace_bytes(64, 32, 128, 4096) == 64 * 32 * 65 * 129 * 4 + 64 * 32 * 4
    assert fi.fi_decode_workspace_bytes(8, 64, 128, 131072) == 8 * 64 * 2049 * 129 * 4 + 8 * 64 * 4
    assert fi.fi_decode_workspace_bytes(1, 4, 64, 1) == 1 * 4 * 2 * 65 * 4 + 4 * 4


def _kv(k_dtype="e4m3", v_dtype=None, *, page=16, hkv=2, d=64, lens=(5, 17), ptrs=False, lpl=None):
    """A paged-KV struct over host arrays; device pointers NULL unless ptrs."""
    lens = np.asarray(lens)
    npg = (lens + page - 1) // page
    indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    last = (lens - (npg - 1) * page).astype(np.int32) if lpl is None else np.asarray(lpl, np.int32)
    s = fi.PagedKV()
    fake = 0x10000 if ptrs else None
    s.k = s.v = fake
    s.k_dtype = fi.DTYPES[k_dtype]
    s.v_dtype = fi.DTYPES[v_dtype or k_dtype]
    s.stride_token = hkv * d
    s.stride_head = d
    s.stride_page = page * hkv * d
    s.num_pages, s.page_size, s.num_kv_heads, s.head_dim = int(indptr[-1]), page, hkv, d
    s.indptr = s.indices = s.last_page_len = fake
    s.indptr_h = indptr.ctypes.data
    s.last_page_len_h = last.ctypes.data
    s.k_scale = s.v_scale = 1.0
    return s, (indptr, last)


def _decode(L, kv, q="f16", o="default", hq=4, batch=2, qp=None, op=None, ws=None, wsb=0, sm=0.0):
    return L.fi_batch_decode_paged(qp, fi.DTYPES[q], batch, hq, ctypes.byref(kv), op, fi.DTYPES[o], None, sm, ws, wsb,
                                   None)


def _prefill(L, kv, q="f16", o="default", hq=4, batch=2, qp=None, op=None):
    qo = np.array([0, 3, 7], np.int32)
    return L.fi_batch_prefill_paged(qp, fi.DTYPES[q], None, qo.ctypes.data, batch, hq, ctypes.byref(kv), 1, op,
                                    fi.DTYPES[o], None, 0.0, None, 0, None)


def _single(L, q="f16", k="e4m3", v=None, o="default", d=64, hq=4, hkv=2, kv_len=8):
    return L.fi_single_decode(None, fi.DTYPES[q], None, None, fi.DTYPES[k], fi.DTYPES[v or k], kv_len, hq, hkv, d,
                              1.0, 1.0, None, fi.DTYPES[o], None, 0.0, None, 0, None)


def _ragged(k_dtype="e4m3", v_dtype=None, *, hkv=2, d=64, lens=(5, 17), lead=0, ptrs=False, num_tokens=None):
    """A ragged-KV struct over host arrays; device pointers NULL unless ptrs."""
    indptr = np.concatenate([[lead], lead + np.cumsum(lens)]).astype(np.int32)
    s = fi.RaggedKV()
    fake = 0x10000 if ptrs else None
    s.k = s.v = fake
    s.k_dtype = fi.DTYPES[k_dtype]
    s.v_dtype = fi.DTYPES[v_dtype or k_dtype]
    s.stride_token, s.stride_head = hkv * d, d
    s.num_tokens = int(indptr[-1]) if num_tokens is None else num_tokens
    s.num_kv_heads, s.head_dim = hkv, d
    s.indptr = fake
    s.indptr_h = indptr.ctypes.data
    s.k_scale = s.v_scale = 1.0
    return s, (indptr,)


def _prefill_ragged(L, kv, q="f16", o="default", hq=4, batch=2, qp=None, op=None, qo_dev=None):
    qo = np.array([0, 3, 7], np.int32)
    return L.fi_batch_prefill_ragged(qp, fi.DTYPES[q], qo_dev, qo.ctypes.data, batch, hq, ctypes.byref(kv), 1, op,
                                     fi.DTYPES[o], None, 0.0, None)


def _single_prefill(L, q="f16", k="e4m3", v=None, o="default", d=64, hq=4, hkv=2, qo_len=5, kv_len=8, qp=None,
                    kp=None, op=None):
    return L.fi_single_prefill(qp, fi.DTYPES[q], qo_len, kp, kp, fi.DTYPES[k], fi.DTYPES[v or k], kv_len, hq, hkv, d,
                               1, 1.0, 1.0, op, fi.DTYPES[o], None, 0.0, None)


def _prefill_fp8q(L, kv, q="e4m3", o="f16", hq=4, batch=2, qp=None, op=None, q_scale=1.0, qo_dev=None):
    qo = np.array([0, 3, 7], np.int32)
    return L.fi_batch_prefill_paged_fp8q(qp, fi.DTYPES[q], q_scale, qo_dev, qo.ctypes.data, batch, hq, ctypes.byref(kv),
                                         1, 0, op, fi.DTYPES[o], None, 0.0, None)


def _ragged_fp8q(L, kv, q="e4m3", o="f16", hq=4, batch=2, qp=None, op=None, q_scale=1.0, qo_dev=None):
    qo = np.array([0, 3, 7], np.int32)
    return L.fi_batch_prefill_ragged_fp8q(qp, fi.DTYPES[q], q_scale, qo_dev, qo.ctypes.data, batch, hq,
                                          ctypes.byref(kv), 1, 1, op, fi.DTYPES[o], None, 0.0, None)


def _single_fp8q(L, q="e4m3", k="e4m3", v=None, o="f16", d=64, hq=4, hkv=2, qo_len=5, kv_len=8, qp=None, kp=None,
                 op=None, q_scale=1.0):
    return L.fi_single_prefill_fp8q(qp, fi.DTYPES[q], q_scale, qo_len, kp, kp, fi.DTYPES[k], fi.DTYPES[v or k], kv_len,
                                    hq, hkv, d, 1, 0, 1.0, 1.0, op, fi.DTYPES[o], None, 0.0, None)


def _err(L):
    return L.fi_last_error().decode()


DTYPE_REFUSALS = [
    # (call, kwargs, status, fragment)
    ("decode", dict(q="e4m3"), 1, "fi_batch_decode_paged: q has dtype float8_e4m3fn; an fp8 query is not supported"),
    ("decode", dict(q="f32"), 1, "q has dtype float32"),
    ("decode", dict(o="e4m3"), 1, "o has dtype float8_e4m3fn; an fp8 output is not supported"),
    ("decode", dict(o="e5m2"), 1, "an fp8 output is not supported"),
    ("decode", dict(o="f32"), 1, "o has dtype float32"),
    ("decode", dict(k="f16", v="bf16"), 1, "fi_batch_decode_paged: k has dtype float16 but v has dtype bfloat16"),
    ("decode", dict(k="e4m3", v="e5m2"), 1, "k has dtype float8_e4m3fn but v has dtype float8_e5m2"),
    ("decode", dict(k="e4m3", v="f16"), 1, "k has dtype float8_e4m3fn but v has dtype float16"),
    ("decode", dict(k="i8"), 1, "KV cache has dtype int8, which has no float interpretation"),
    ("decode", dict(k="u8"), 1, "KV cache has dtype uint8, which has no float interpretation"),
    ("decode", dict(k="f32"), 1, "KV cache has dtype float32"),
    ("prefill", dict(q="f16", k="bf16"), 1,
     "fi_batch_prefill_paged: q has dtype float16 but the KV cache has dtype bfloat16; prefill needs a 2-byte KV"),
    ("prefill", dict(q="bf16", k="f16"), 1, "q has dtype bfloat16 but the KV cache has dtype float16"),
    ("prefill", dict(q="e5m2"), 1, "an fp8 query is not supported"),
    ("prefill", dict(k="f16", v="bf16"), 1, "k has dtype float16 but v has dtype bfloat16"),
    ("prefill", dict(k="i8"), 1, "no float interpretation"),
    ("prefill", dict(o="e4m3"), 1, "an fp8 output is not supported"),
    ("single", dict(k="f16", v="bf16"), 1, "fi_single_decode: k has dtype float16 but v has dtype bfloat16"),
    ("single", dict(k="u8"), 1, "fi_single_decode: KV cache has dtype uint8"),
    ("single", dict(o="e4m3"), 1, "fi_single_decode: o has dtype float8_e4m3fn"),
    ("single", dict(q="e4m3"), 1, "fi_single_decode: q has dtype float8_e4m3fn"),
    ("ragged", dict(q="f16", k="bf16"), 1,
     "fi_batch_prefill_ragged: q has dtype float16 but the KV cache has dtype bfloat16; prefill needs a 2-byte KV"),
    ("ragged", dict(k="e4m3", v="e5m2"), 1, "fi_batch_prefill_ragged: k has dtype float8_e4m3fn but v has dtype"),
    ("ragged", dict(k="i8"), 1, "fi_batch_prefill_ragged: KV cache has dtype int8, which has no float interpretation"),
    ("ragged", dict(q="e4m3"), 1, "fi_batch_prefill_ragged: q has dtype float8_e4m3fn; an fp8 query"),
    ("ragged", dict(o="e5m2"), 1, "fi_batch_prefill_ragged: o has dtype float8_e5m2"),
    ("single_prefill", dict(q="bf16", k="f16"), 1,
     "fi_single_prefill: q has dtype bfloat16 but the KV cache has dtype float16"),
    ("single_prefill", dict(k="f16", v="bf16"), 1, "fi_single_prefill: k has dtype float16 but v has dtype bfloat16"),
    ("single_prefill", dict(k="f32"), 1, "fi_single_prefill: KV cache has dtype float32"),
    ("single_prefill", dict(o="e4m3"), 1, "fi_single_prefill: o has dtype float8_e4m3fn"),
    ("fp8q", dict(q="f16", o="f16"), 1, "fi_batch_prefill_paged_fp8q: q has dtype float16; this call takes an fp8 query"),
    ("fp8q", dict(q="e4m3fnuz", o="f16"), 1, "q has dtype float8_e4m3fnuz; this call takes an fp8 query"),
    ("fp8q", dict(q="e4m3", o="default"), 1, "o_dtype must be given for an fp8 query"),
    ("fp8q", dict(q="e4m3", o="e5m2"), 1, "o has dtype float8_e5m2; an fp8 output is not supported"),
    ("fp8q", dict(q="e5m2", o="bf16", k="e4m3", v="e5m2"), 1, "k has dtype float8_e4m3fn but v has dtype float8_e5m2"),
    ("fp8q", dict(q="e4m3", o="f16", k="f16"), 1,
     "q has dtype float8_e4m3fn but the KV cache has dtype float16; an fp8 query needs an fp8 KV cache"),
    ("fp8q", dict(q="e4m3", o="f16", k="u8"), 1, "KV cache has dtype uint8, which has no float interpretation"),
    ("fp8q", dict(q="e4m3", o="f16", k="e5m2fnuz"), 1,
     "float8_e5m2fnuz, the gfx942 fnuz variant; an fp8-query prefill runs the OCP fp8 matrix cores"),
    ("fp8q", dict(q="e5m2", o="bf16", k="e4m3fnuz"), 1, "float8_e4m3fnuz, the gfx942 fnuz variant"),
    ("ragged_fp8q", dict(q="f16", o="f16"), 1, "fi_batch_prefill_ragged_fp8q: q has dtype float16; this call takes an"),
    ("ragged_fp8q", dict(q="e4m3", o="default"), 1, "fi_batch_prefill_ragged_fp8q: o_dtype must be given"),
    ("ragged_fp8q", dict(q="e4m3", o="f16", k="e4m3fnuz"), 1, "float8_e4m3fnuz, the gfx942 fnuz variant"),
    ("ragged_fp8q", dict(q="e4m3", o="f16", k="bf16"), 1, "an fp8 query needs an fp8 KV cache"),
    ("ragged_fp8q", dict(q="e5m2", o="e4m3"), 1, "an fp8 output is not supported"),
    ("single_fp8q", dict(q="bf16", o="bf16"), 1, "fi_single_prefill_fp8q: q has dtype bfloat16; this call takes an"),
    ("single_fp8q", dict(q="e4m3", o="f16", k="e4m3", v="e5m2"), 1, "k has dtype float8_e4m3fn but v has dtype"),
    ("single_fp8q", dict(q="e4m3", o="f16", k="e5m2fnuz"), 1, "fi_single_prefill_fp8q: KV cache has dtype "
     "float8_e5m2fnuz, the gfx942 fnuz variant"),
    ("single_fp8q", dict(q="e4m3", o="f16", k="i8"), 1, "no float interpretation"),
]


@no_gpu
@pytest.mark.parametrize("call,kw,status,frag", DTYPE_REFUSALS, ids=[f"{c}-{i}" for i, (c, *_r) in enumerate(DTYPE_REFUSALS)])
def test_dtype_refusals(L, call, kw, status, frag):
    k = kw.get("k", "e4m3")
    v = kw.get("v", k)
    q = kw.get("q", "f16")
    o = kw.get("o", "default")
    if call == "single":
        st = _single(L, q=q, k=k, v=v, o=o)
    elif call == "single_prefill":
        st = _single_prefill(L, q=q, k=k, v=v, o=o)
    elif call == "fp8q":
        kv, keep = _kv(k, v)
        st = _prefill_fp8q(L, kv, q=q, o=o)
    elif call == "ragged_fp8q":
        kv, keep = _ragged(k, v)
        st = _ragged_fp8q(L, kv, q=q, o=o)
    elif call == "single_fp8q":
        st = _single_fp8q(L, q=q, k=k, v=v, o=o)
    elif call == "ragged":
        kv, keep = _ragged(k, v)
        st = _prefill_ragged(L, kv, q=q, o=o)
    else:
        kv, keep = _kv(k, v)
        st = _decode(L, kv, q=q, o=o) if call == "decode" else _prefill(L, kv, q=q, o=o)
    assert st == status
    assert frag in _err(L), _err(L)


@no_gpu
def test_decode_accepts_mixed_2byte_before_pointer_checks(L):
    """Decode admits a 2-byte KV that differs from q ("fp8 KV cache in the
    in-tree prefill kernel", Architecture / design notes): with NULL pointers
    the first refusal is the pointer check, not a dtype refusal."""
    for q, k in (("f16", "bf16"), ("bf16", "f16")):
        kv, keep = _kv(k)
        st = _decode(L, kv, q=q)
        assert st == 3 and "must not be NULL" in _err(L), _err(L)


@no_gpu
def test_decode_accepts_fnuz_before_pointer_checks(L):
    """fnuz caches pass the decode dtype checks (the next refusal is the NULL
    pointer), in the batch and the single call."""
    for k in ("e4m3fnuz", "e5m2fnuz"):
        kv, keep = _kv(k)
        assert _decode(L, kv) == 3 and "must not be NULL" in _err(L), _err(L)
        assert _single(L, k=k) == 3 and "must not be NULL" in _err(L), _err(L)


@no_gpu
def test_prefill_accepts_fnuz_before_pointer_checks(L):
    """fnuz caches pass the dtype checks of the prefill calls that take a
    2-byte query -- paged, ragged and single (the next refusal is the NULL
    pointer) -- while the fp8-query prefill refuses them."""
    for k in ("e4m3fnuz", "e5m2fnuz"):
        for q in ("f16", "bf16"):
            kv, keep = _kv(k)
            assert _prefill(L, kv, q=q) == 3 and "must not be NULL" in _err(L), _err(L)
            kr, keepr = _ragged(k, k)
            assert _prefill_ragged(L, kr, q=q) == 3 and "must not be NULL" in _err(L), _err(L)
            assert _single_prefill(L, q=q, k=k, v=k) == 3 and "must not be NULL" in _err(L), _err(L)


@no_gpu
def test_ragged_and_single_fp8q_reach_pointer_checks(L):
    """Valid fp8-query ragged and single calls pass every dtype, shape and
    scale check and stop at the NULL pointers; a bad q_scale is refused first."""
    kv, keep = _ragged("e5m2")
    assert _ragged_fp8q(L, kv) == 3 and "must not be NULL" in _err(L), _err(L)
    assert _ragged_fp8q(L, kv, q_scale=0.0, qo_dev=0x10000) == 3 and "q_scale=0 must be finite and > 0" in _err(L), \
        _err(L)
    assert _single_fp8q(L, k="e5m2") == 3 and "must not be NULL" in _err(L), _err(L)
    assert _single_fp8q(L, q_scale=float("nan")) == 3 and "q_scale=nan" in _err(L), _err(L)


@no_gpu
def test_order_dtype_before_shape(L):
    kv, keep = _kv("i8", d=96)  # both an int8 KV and a bad head_dim: dtype is reported
    assert _decode(L, kv) == 1 and "int8" in _err(L)


@no_gpu
@pytest.mark.parametrize("case", ["head_dim", "heads_ratio", "page_size", "batch"])
def test_shape_refusals(L, case):
    if case == "head_dim":
        kv, keep = _kv(d=96)
        st, frag = _decode(L, kv), "head_dim=96"
    elif case == "heads_ratio":
        kv, keep = _kv(hkv=3)
        st, frag = _decode(L, kv, hq=4), "num_qo_heads=4 is not a multiple of num_kv_heads=3"
    elif case == "page_size":
        kv, keep = _kv(page=16)
        kv.page_size = 12
        st, frag = _decode(L, kv, qp=0x10000, op=0x10000), "page_size=12"
    else:
        kv, keep = _kv()
        st, frag = _decode(L, kv, batch=-1), "batch=-1 is outside"
    assert st == 2, _err(L)
    assert frag in _err(L)


@no_gpu
def test_argument_refusals(L):
    kv, keep = _kv(ptrs=True)
    assert _decode(L, kv, qp=0x10008, op=0x10000) == 3 and "16-byte aligned" in _err(L)
    kv2, keep2 = _kv(ptrs=True, lpl=[5, 0])
    assert _decode(L, kv2, qp=0x10000, op=0x10000) == 3 and "last_page_len[1]=0" in _err(L)
    kv3, keep3 = _kv(ptrs=True, lpl=[17, 1])
    assert _decode(L, kv3, qp=0x10000, op=0x10000) == 3 and "last_page_len[0]=17" in _err(L)
    kv4, keep4 = _kv(ptrs=True)
    kv4.k_scale = float("nan")
    assert _decode(L, kv4, qp=0x10000, op=0x10000) == 3 and "k_scale" in _err(L)
    kv5, keep5 = _kv(ptrs=True)
    kv5.v_scale = 0.0
    assert _decode(L, kv5, qp=0x10000, op=0x10000) == 3 and "v_scale" in _err(L)
    kv6, keep6 = _kv(ptrs=True)
    kv6.stride_token = 2 * 64 + 4  # fp8 rows no longer 16-byte aligned
    assert _decode(L, kv6, qp=0x10000, op=0x10000) == 3 and "16-byte aligned rows" in _err(L)


@no_gpu
def test_stride_limits(L):
    """Byte strides are positive and below 4 GiB (the kernels form gather
    offsets with 32 x 32 -> 64-bit products), for the paged and ragged calls."""
    fake = 0x10000
    kv, keep = _kv(ptrs=True)
    kv.stride_page = 1 << 32  # fp8: one byte per element
    assert _decode(L, kv, qp=fake, op=fake) == 2 and "below 4 GiB" in _err(L)
    kv, keep = _kv(ptrs=True, k_dtype="f16")
    kv.stride_token = 1 << 31  # 2 bytes per element: 4 GiB
    assert _decode(L, kv, qp=fake, op=fake) == 2 and "below 4 GiB" in _err(L)
    kv, keep = _kv(ptrs=True)
    kv.stride_head = 0
    assert _decode(L, kv, qp=fake, op=fake) == 2 and "strides must be positive" in _err(L)
    kv, keep = _kv(ptrs=True)
    kv.stride_page = (1 << 32) - 16  # the largest aligned stride passes every check; the launch then finds no GPU
    assert _decode(L, kv, qp=fake, op=fake) == 5 and "no ROCm-capable device" in _err(L)
    kv, keep = _ragged(ptrs=True)
    kv.stride_head = 1 << 32
    assert _prefill_ragged(L, kv, qp=fake, op=fake, qo_dev=fake) == 2 and "below 4 GiB" in _err(L)


@no_gpu
def test_ragged_and_single_prefill_refusals(L):
    fake = 0x10000
    kv, keep = _ragged()
    assert _prefill_ragged(L, kv, qp=fake, op=fake, qo_dev=fake) == 3 and "k and v must not be NULL" in _err(L)
    kv, keep = _ragged(ptrs=True, num_tokens=20)  # indptr ends at 22
    assert _prefill_ragged(L, kv, qp=fake, op=fake, qo_dev=fake) == 3 and "indptr[2]=22 exceeds num_tokens=20" in _err(L)
    kv, keep = _ragged(ptrs=True, lens=(5, -2))
    assert _prefill_ragged(L, kv, qp=fake, op=fake, qo_dev=fake) == 3 and "indptr is decreasing at request 1" in _err(L)
    kv, keep = _ragged(ptrs=True)
    kv.indptr = None
    assert _prefill_ragged(L, kv, qp=fake, op=fake, qo_dev=fake) == 3 and "indptr (device)" in _err(L)
    kv, keep = _ragged(ptrs=True)
    assert _prefill_ragged(L, kv, qp=fake, op=fake) == 3 and "qo_indptr and qo_indptr_h" in _err(L)
    kv, keep = _ragged(ptrs=True, d=96)
    assert _prefill_ragged(L, kv, qp=fake, op=fake, qo_dev=fake) == 2 and "head_dim=96" in _err(L)
    kv, keep = _ragged(ptrs=True)
    kv.stride_token = 2 * 64 + 4
    assert _prefill_ragged(L, kv, qp=fake, op=fake, qo_dev=fake) == 3 and "16-byte aligned rows" in _err(L)
    kv, keep = _ragged(ptrs=True)
    kv.k_scale = float("inf")
    assert _prefill_ragged(L, kv, qp=fake, op=fake, qo_dev=fake) == 3 and "k_scale" in _err(L)
    assert _single_prefill(L, qo_len=-1) == 2 and "qo_len=-1 is negative" in _err(L)
    assert _single_prefill(L, kv_len=1 << 30) == 2 and "kv_len=1073741824" in _err(L)
    assert _single_prefill(L, qp=fake, op=fake) == 3 and "k and v must not be NULL" in _err(L)
    assert _single_prefill(L, qp=fake + 8, op=fake, kp=fake) == 3 and "16-byte aligned" in _err(L)
    assert _single_prefill(L, hq=6, hkv=4) == 2 and "num_qo_heads=6 is not a multiple" in _err(L)
    # nothing to compute: accepted without touching the device
    assert _single_prefill(L, qo_len=0, kv_len=0) == 0
    kv, keep = _ragged(ptrs=True)
    assert L.fi_batch_prefill_ragged(None, 1, None, None, 0, 4, ctypes.byref(kv), 1, None, 0, None, 0.0, None) == 0


def _decode_fp8q(L, kv, q="e4m3", o="f16", hq=4, batch=2, qp=None, op=None, q_scale=1.0):
    return L.fi_batch_decode_paged_fp8q(qp, fi.DTYPES[q], q_scale, batch, hq, ctypes.byref(kv), op, fi.DTYPES[o], None,
                                        0.0, None, 0, None)


@no_gpu
def test_decode_fp8q_refusals(L):
    kv, keep = _kv("e4m3")
    assert _decode_fp8q(L, kv, q="bf16") == 1 and "fi_batch_decode_paged_fp8q: q has dtype bfloat16" in _err(L)
    assert _decode_fp8q(L, kv, o="default") == 1 and "o_dtype must be given for an fp8 query" in _err(L)
    assert _decode_fp8q(L, kv, o="e4m3") == 1 and "an fp8 output is not supported" in _err(L)
    kv2, keep2 = _kv("f16")
    assert _decode_fp8q(L, kv2) == 1 and "an fp8 query needs an fp8 KV cache" in _err(L)
    kv3, keep3 = _kv("e4m3", "e5m2")
    assert _decode_fp8q(L, kv3) == 1 and "k has dtype float8_e4m3fn but v has dtype float8_e5m2" in _err(L)
    kv4, keep4 = _kv("e5m2fnuz")  # fnuz passes the dtype checks in decode
    assert _decode_fp8q(L, kv4) == 3 and "must not be NULL" in _err(L)
    assert _decode_fp8q(L, kv, qp=0x10000, op=0x10000, q_scale=-1.0) == 3 and "q_scale=-1" in _err(L)
    kv5, keep5 = _kv("e4m3", d=48)
    assert _decode_fp8q(L, kv5) == 2 and "head_dim=48" in _err(L)


@no_gpu
def test_fp8q_argument_refusals(L):
    fake = 0x10000
    kv, keep = _kv(ptrs=True)
    assert _prefill_fp8q(L, kv, qp=fake, op=fake, q_scale=0.0, qo_dev=fake) == 3 and "q_scale=0" in _err(L)
    assert _prefill_fp8q(L, kv, qp=fake, op=fake, q_scale=float("nan"), qo_dev=fake) == 3 and "q_scale" in _err(L)
    assert _prefill_fp8q(L, kv, qp=fake, op=fake) == 3 and "qo_indptr and qo_indptr_h" in _err(L)
    assert _prefill_fp8q(L, kv, qp=fake + 4, op=fake, qo_dev=fake) == 3 and "16-byte aligned" in _err(L)
    kv2, keep2 = _kv(ptrs=True, d=80)
    assert _prefill_fp8q(L, kv2, qp=fake, op=fake, qo_dev=fake) == 2 and "head_dim=80" in _err(L)
    kv3, keep3 = _kv(ptrs=True, lpl=[5, 0])
    assert _prefill_fp8q(L, kv3, qp=fake, op=fake, qo_dev=fake) == 3 and "last_page_len[1]=0" in _err(L)
    assert _prefill_fp8q(L, kv, batch=0) == 0


@no_gpu
def test_workspace_too_small(L, monkeypatch):
    monkeypatch.setenv("FI_SPLIT_KV", "128")
    kv, keep = _kv(ptrs=True, lens=(1000, 300))
    st = _decode(L, kv, qp=0x10000, op=0x10000, ws=0x10000, wsb=16)
    assert st == 4 and "workspace_bytes=16" in _err(L), _err(L)


def test_scratch_size_matches_header():
    m = re.search(r"#define FI_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == fi.DECODE_SCRATCH_BYTES


@no_gpu
def test_noalloc_refuses_a_split_beyond_its_scratch(L, monkeypatch):
    """A split whose partial states exceed the allocation-free call's scratch
    is refused with FI_E_WORKSPACE before any HIP call; the dtype refusals come
    first, as in fi_batch_decode_paged."""
    monkeypatch.setenv("FI_SPLIT_KV", "64")
    kv, keep = _kv(ptrs=True, hkv=8, d=128, lens=(70000, 10))  # 1094 pieces x 64 heads x 129 floats x 2
    fake = 0x10000
    st = L.fi_batch_decode_paged_noalloc(fake, fi.DTYPES["f16"], 2, 64, ctypes.byref(kv), fake, 0, None, 0.0, None)
    assert st == 4 and "allocation-free call holds at most 33554432 bytes" in _err(L), _err(L)
    kv2, keep2 = _kv("e4m3", "e5m2", ptrs=True)
    st = L.fi_batch_decode_paged_noalloc(fake, fi.DTYPES["f16"], 2, 4, ctypes.byref(kv2), fake, 0, None, 0.0, None)
    assert st == 1 and "fi_batch_decode_paged_noalloc: k has dtype float8_e4m3fn but v has dtype float8_e5m2" in _err(L)
    st = L.fi_batch_decode_paged_noalloc(fake, fi.DTYPES["f16"], 2, 4, ctypes.byref(kv2), fake, fi.DTYPES["e4m3"],
                                         None, 0.0, None)
    assert st == 1 and "an fp8 output is not supported" in _err(L)


def _pod(L, kv_p, kv_d, q="f16", o="default", hq=4, batch_p=2, batch_d=2, ptrs=False, qo=(0, 3, 7)):
    qo = np.asarray(qo, np.int32)
    fake = 0x10000 if ptrs else None
    return L.fi_batch_pod_paged(fake, fake, qo.ctypes.data, batch_p, ctypes.byref(kv_p), 1, fake, None, fake, batch_d,
                                ctypes.byref(kv_d), fake, None, fi.DTYPES[q], fi.DTYPES[o], hq, 0.0, None, 0, None)


@no_gpu
def test_pod_refusals(L):
    """The POD call: the prefill rules on both phases (sentences naming the
    decode phase when it is the decode phase's), then the cross-phase checks
    -- one KV dtype and one head layout for both phases, never reinterpreted
    ("fp8 KV cache in the in-tree prefill kernel", review comments on POD
    cross-phase dtype validation) -- then shapes and the argument budget."""
    kv, keep = _kv(ptrs=True)
    assert _pod(L, kv, kv, q="e4m3", ptrs=True) == 1 and "q has dtype float8_e4m3fn" in _err(L)
    assert _pod(L, kv, kv, o="e5m2", ptrs=True) == 1 and "an fp8 output is not supported" in _err(L)
    kvm, keepm = _kv("e4m3", "e5m2", ptrs=True)
    assert _pod(L, kvm, kv, ptrs=True) == 1 and _err(L).startswith("fi_batch_pod_paged: k has dtype")
    assert _pod(L, kv, kvm, ptrs=True) == 1
    assert _err(L).startswith("fi_batch_pod_paged (decode phase): k has dtype float8_e4m3fn but v has dtype float8_e5m2")
    kvb, keepb = _kv("bf16", ptrs=True)
    assert _pod(L, kvb, kvb, q="f16", ptrs=True) == 1 and "prefill needs a 2-byte KV cache of the query's dtype" in _err(L)
    kvi, keepi = _kv("i8", ptrs=True)
    assert _pod(L, kv, kvi, ptrs=True) == 1 and "(decode phase): KV cache has dtype int8" in _err(L)
    kv5, keep5 = _kv("e5m2", ptrs=True)
    assert _pod(L, kv, kv5, ptrs=True) == 1
    assert "prefill phase's KV cache has dtype float8_e4m3fn but the decode phase's has dtype float8_e5m2" in _err(L)
    kvh, keeph = _kv(ptrs=True, hkv=4)
    assert _pod(L, kv, kvh, ptrs=True) == 2 and "both phases share the head layout" in _err(L)
    assert _pod(L, kv, kv, hq=3, ptrs=True) == 2 and "not a multiple" in _err(L)
    assert _pod(L, kv, kv, batch_p=-1, ptrs=True) == 2
    kvl, keepl = _kv(ptrs=True, lpl=[5, 0])
    assert _pod(L, kv, kvl, ptrs=True) == 3 and "(decode phase): last_page_len[1]=0" in _err(L)
    assert _pod(L, kv, kv, ptrs=False) == 3  # NULL pointers
    # more (request, query block) pairs than one launch's arguments carry:
    # 449 requests of 40 queries (4 q heads, 1 kv head group -> 64 rows per pair)
    lens = np.full(449, 40)
    kvp, keepp = _kv(ptrs=True, lens=lens)
    qo = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    assert _pod(L, kvp, kv, batch_p=449, ptrs=True, qo=qo) == 2
    assert "more than 384 (request, query block) pairs" in _err(L), _err(L)


@no_gpu
def test_widen_refusals(L):
    assert L.fi_fp8_widen(None, 4, fi.DTYPES["f16"], fi.DTYPES["f16"], None, None) == 1
    assert "src has dtype float16" in _err(L)
    assert L.fi_fp8_widen(None, 4, fi.DTYPES["e4m3fnuz"], fi.DTYPES["f16"], None, None) == 3  # fnuz passes dtypes
    assert L.fi_fp8_widen(None, 4, fi.DTYPES["e4m3"], fi.DTYPES["e4m3"], None, None) == 1
    assert L.fi_fp8_widen(None, 4, fi.DTYPES["e4m3"], fi.DTYPES["bf16"], None, None) == 3
    assert L.fi_fp8_widen(None, 0, fi.DTYPES["e4m3"], fi.DTYPES["bf16"], None, None) == 0


def test_python_error_classes():
    assert issubclass(fi.FiValueError, ValueError)
    assert issubclass(fi.FiRuntimeError, RuntimeError)
