"""Python binding of libfi.so (include/fi.h): argument marshalling only.

Every computation happens in the HIP library; this module turns torch tensors
(device memory) into the pointers, dtypes, strides and the stream the C calls
take, and turns a non-zero fi_status into an exception.  If libfi.so has not
been built the first call raises; there is no fallback path.

Errors mirror the split the pages describe for refusals: a refused dtype,
shape, argument or workspace raises FiValueError (a ValueError); a HIP runtime
failure raises FiRuntimeError (a RuntimeError) ("fp8 KV cache in the in-tree
prefill kernel", AMD-Ecosystem/flashinfer PR #368, Architecture / design
notes on where each refusal surfaces).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FI_LIB_PATH names another build of the same library (the sanitizer build's
# CPU checks use it); by default the in-tree libfi.so.
LIB_PATH = os.environ.get("FI_LIB_PATH") or os.path.join(_HERE, "libfi.so")

# fi_dtype
DTYPES = {
    "default": 0, "f16": 1, "bf16": 2, "e4m3": 3, "e5m2": 4, "f32": 5, "i8": 6, "u8": 7,
    "e4m3fnuz": 8, "e5m2fnuz": 9,
}
TORCH_DTYPES = {
    torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "e4m3", torch.float8_e5m2: "e5m2",
    torch.float32: "f32", torch.int8: "i8", torch.uint8: "u8", torch.float8_e4m3fnuz: "e4m3fnuz",
    torch.float8_e5m2fnuz: "e5m2fnuz",
}
STATUS = {0: "FI_OK", 1: "FI_E_DTYPE", 2: "FI_E_SHAPE", 3: "FI_E_ARG", 4: "FI_E_WORKSPACE", 5: "FI_E_HIP"}

# every symbol include/fi.h declares
EXPORTS = ("fi_last_error", "fi_decode_workspace_bytes", "fi_batch_decode_paged", "fi_batch_decode_paged_fp8q",
           "fi_batch_prefill_paged", "fi_batch_prefill_paged_fp8q", "fi_batch_prefill_ragged",
           "fi_batch_prefill_ragged_fp8q", "fi_single_prefill", "fi_single_prefill_fp8q", "fi_single_decode",
           "fi_fp8_widen", "fi_batch_decode_paged_noalloc", "fi_batch_pod_paged")
DECODE_SCRATCH_BYTES = 32 << 20  # FI_DECODE_SCRATCH_BYTES


class FiError(Exception):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{STATUS.get(status, status)}] {message}")
        self.status = status
        self.message = message


class FiValueError(FiError, ValueError):
    pass


class FiRuntimeError(FiError, RuntimeError):
    pass


class PagedKV(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_dtype", ctypes.c_int), ("v_dtype", ctypes.c_int),
        ("stride_page", ctypes.c_int64), ("stride_token", ctypes.c_int64), ("stride_head", ctypes.c_int64),
        ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("indptr", ctypes.c_void_p), ("indices", ctypes.c_void_p), ("last_page_len", ctypes.c_void_p),
        ("indptr_h", ctypes.c_void_p), ("last_page_len_h", ctypes.c_void_p),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
    ]


class RaggedKV(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_dtype", ctypes.c_int), ("v_dtype", ctypes.c_int),
        ("stride_token", ctypes.c_int64), ("stride_head", ctypes.c_int64),
        ("num_tokens", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("indptr", ctypes.c_void_p), ("indptr_h", ctypes.c_void_p),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfi.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_paged_fp8_amd.build` "
                           "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz, en = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t,
                                 ctypes.c_int)
    L.fi_last_error.restype = ctypes.c_char_p
    L.fi_last_error.argtypes = []
    L.fi_decode_workspace_bytes.restype = sz
    L.fi_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.fi_batch_decode_paged.restype = en
    L.fi_batch_decode_paged.argtypes = [vp, en, i32, i32, ctypes.POINTER(PagedKV), vp, en, vp, f32, vp, sz, vp]
    L.fi_batch_decode_paged_noalloc.restype = en
    L.fi_batch_decode_paged_noalloc.argtypes = [vp, en, i32, i32, ctypes.POINTER(PagedKV), vp, en, vp, f32, vp]
    L.fi_batch_pod_paged.restype = en
    L.fi_batch_pod_paged.argtypes = [vp, vp, vp, i32, ctypes.POINTER(PagedKV), i32, vp, vp, vp, i32,
                                     ctypes.POINTER(PagedKV), vp, vp, en, en, i32, f32, vp, sz, vp]
    L.fi_batch_decode_paged_fp8q.restype = en
    L.fi_batch_decode_paged_fp8q.argtypes = [vp, en, f32, i32, i32, ctypes.POINTER(PagedKV), vp, en, vp, f32, vp, sz,
                                             vp]
    L.fi_batch_prefill_paged.restype = en
    L.fi_batch_prefill_paged.argtypes = [vp, en, vp, vp, i32, i32, ctypes.POINTER(PagedKV), i32, vp, en, vp, f32, vp,
                                         sz, vp]
    L.fi_batch_prefill_paged_fp8q.restype = en
    L.fi_batch_prefill_paged_fp8q.argtypes = [vp, en, f32, vp, vp, i32, i32, ctypes.POINTER(PagedKV), i32, i32, vp, en,
                                              vp, f32, vp]
    L.fi_batch_prefill_ragged.restype = en
    L.fi_batch_prefill_ragged.argtypes = [vp, en, vp, vp, i32, i32, ctypes.POINTER(RaggedKV), i32, vp, en, vp, f32,
                                          vp]
    L.fi_batch_prefill_ragged_fp8q.restype = en
    L.fi_batch_prefill_ragged_fp8q.argtypes = [vp, en, f32, vp, vp, i32, i32, ctypes.POINTER(RaggedKV), i32, i32, vp,
                                               en, vp, f32, vp]
    L.fi_single_prefill_fp8q.restype = en
    L.fi_single_prefill_fp8q.argtypes = [vp, en, f32, i32, vp, vp, en, en, i32, i32, i32, i32, i32, i32, f32, f32, vp,
                                         en, vp, f32, vp]
    L.fi_single_prefill.restype = en
    L.fi_single_prefill.argtypes = [vp, en, i32, vp, vp, en, en, i32, i32, i32, i32, i32, f32, f32, vp, en, vp, f32,
                                    vp]
    L.fi_single_decode.restype = en
    L.fi_single_decode.argtypes = [vp, en, vp, vp, en, en, i32, i32, i32, i32, f32, f32, vp, en, vp, f32, vp, sz, vp]
    L.fi_fp8_widen.restype = en
    L.fi_fp8_widen.argtypes = [vp, i64, en, en, vp, vp]
    _lib = L
    return L


def check(status: int) -> None:
    if status == 0:
        return
    msg = lib().fi_last_error().decode()
    if status == 5:
        raise FiRuntimeError(status, msg)
    raise FiValueError(status, msg)


def _dt(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if isinstance(x, torch.dtype):
        return DTYPES[TORCH_DTYPES[x]]
    return DTYPES[x]


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr() if isinstance(t, torch.Tensor) else int(t)


def _stream(stream, *tensors):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _host_i32(t):
    """Host int32 copy of an index array (kept alive by the caller's frame)."""
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.int32).contiguous()
    return torch.as_tensor(t, dtype=torch.int32).contiguous()


def fi_decode_workspace_bytes(batch: int, num_qo_heads: int, head_dim: int, max_kv_len: int) -> int:
    return int(lib().fi_decode_workspace_bytes(batch, num_qo_heads, head_dim, max_kv_len))


def make_paged_kv(k_pool, v_pool, indptr, indices, last_page_len, *, k_scale=1.0, v_scale=1.0, kv_dtype=None,
                  k_dtype=None, v_dtype=None, indptr_h=None, last_page_len_h=None):
    """Describe a paged cache.  Pools are [num_pages, page_size, H_kv, head_dim]
    tensors with a contiguous last dimension; raw fp8 may be passed as uint8
    with kv_dtype naming the format.  Returns (struct, keepalive): the struct
    holds raw pointers, and keepalive holds every tensor they point at (the
    pools, the device page table and the host copies), so the caller keeps
    keepalive for as long as the struct is used."""
    if tuple(k_pool.stride()) != tuple(v_pool.stride()) or k_pool.shape != v_pool.shape:
        raise FiValueError(2, "k and v pools must have the same shape and strides")
    kd = k_dtype if k_dtype is not None else (kv_dtype if kv_dtype is not None else k_pool.dtype)
    vd = v_dtype if v_dtype is not None else (kv_dtype if kv_dtype is not None else v_pool.dtype)
    ih = _host_i32(indptr_h if indptr_h is not None else indptr)
    lh = _host_i32(last_page_len_h if last_page_len_h is not None else last_page_len)
    s = PagedKV()
    s.k, s.v = _ptr(k_pool), _ptr(v_pool)
    s.k_dtype, s.v_dtype = _dt(kd), _dt(vd)
    s.stride_page, s.stride_token, s.stride_head = k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)
    s.num_pages, s.page_size, s.num_kv_heads, s.head_dim = (int(k_pool.shape[0]), int(k_pool.shape[1]),
                                                            int(k_pool.shape[2]), int(k_pool.shape[3]))
    s.indptr, s.indices, s.last_page_len = _ptr(indptr), _ptr(indices), _ptr(last_page_len)
    s.indptr_h, s.last_page_len_h = ih.data_ptr(), lh.data_ptr()
    s.k_scale, s.v_scale = float(k_scale), float(v_scale)
    return s, (ih, lh, k_pool, v_pool, indptr, indices, last_page_len)


def fi_batch_decode_paged(q, kv: PagedKV, o, *, q_dtype=None, o_dtype=None, lse=None, sm_scale=0.0,
                          workspace=None, workspace_bytes=None, batch=None, num_qo_heads=None, stream=None):
    """q [batch, H_qo, D] and o [batch, H_qo, D] device tensors."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    st = lib().fi_batch_decode_paged(
        _ptr(q), _dt(q_dtype if q_dtype is not None else q.dtype),
        int(batch if batch is not None else q.shape[0]), int(num_qo_heads if num_qo_heads is not None else q.shape[1]),
        ctypes.byref(kv), _ptr(o), _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse), float(sm_scale),
        _ptr(workspace), int(workspace_bytes), _stream(stream, q, o))
    check(st)
    return o


def fi_batch_decode_paged_noalloc(q, kv: PagedKV, o, *, q_dtype=None, o_dtype=None, lse=None, sm_scale=0.0,
                                  batch=None, num_qo_heads=None, stream=None):
    """fi_batch_decode_paged with the split-KV state in the library's own
    per-device scratch (no workspace argument, nothing allocated)."""
    st = lib().fi_batch_decode_paged_noalloc(
        _ptr(q), _dt(q_dtype if q_dtype is not None else q.dtype),
        int(batch if batch is not None else q.shape[0]), int(num_qo_heads if num_qo_heads is not None else q.shape[1]),
        ctypes.byref(kv), _ptr(o), _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse), float(sm_scale),
        _stream(stream, q, o))
    check(st)
    return o


def fi_batch_decode_paged_fp8q(q, kv: PagedKV, o, *, q_dtype, o_dtype=None, q_scale=1.0, lse=None, sm_scale=0.0,
                               workspace=None, workspace_bytes=None, batch=None, num_qo_heads=None, stream=None):
    """q [batch, H_qo, D] fp8 codes (a float8 tensor, or uint8 with q_dtype naming
    the format); o [batch, H_qo, D] float16 or bfloat16."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    st = lib().fi_batch_decode_paged_fp8q(
        _ptr(q), _dt(q_dtype), float(q_scale), int(batch if batch is not None else q.shape[0]),
        int(num_qo_heads if num_qo_heads is not None else q.shape[1]), ctypes.byref(kv), _ptr(o),
        _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse), float(sm_scale), _ptr(workspace),
        int(workspace_bytes), _stream(stream, q, o))
    check(st)
    return o


def fi_batch_prefill_paged(q, qo_indptr, kv: PagedKV, o, *, causal=True, q_dtype=None, o_dtype=None, lse=None,
                           sm_scale=0.0, qo_indptr_h=None, batch=None, num_qo_heads=None, workspace=None,
                           workspace_bytes=0, stream=None):
    """q and o [total_q, H_qo, D]; qo_indptr [batch+1] int32 (device)."""
    qh = _host_i32(qo_indptr_h if qo_indptr_h is not None else qo_indptr)
    st = lib().fi_batch_prefill_paged(
        _ptr(q), _dt(q_dtype if q_dtype is not None else q.dtype), _ptr(qo_indptr), qh.data_ptr(),
        int(batch if batch is not None else qh.numel() - 1), int(num_qo_heads if num_qo_heads is not None else q.shape[1]),
        ctypes.byref(kv), 1 if causal else 0, _ptr(o), _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse),
        float(sm_scale), _ptr(workspace), int(workspace_bytes), _stream(stream, q, o))
    check(st)
    return o


def fi_batch_pod_paged(q_p, qo_indptr, kv_p: PagedKV, o_p, q_d, kv_d: PagedKV, o_d, *, causal=True, lse_p=None,
                       lse_d=None, q_dtype=None, o_dtype=None, sm_scale=0.0, qo_indptr_h=None, batch_p=None,
                       batch_d=None, num_qo_heads=None, workspace=None, workspace_bytes=None, stream=None):
    """One launch over a prefill batch (q_p / o_p [total_q, H_qo, D], qo_indptr
    [batch_p+1] on the device) and a decode batch (q_d / o_d [batch_d, H_qo, D])."""
    qh = _host_i32(qo_indptr_h if qo_indptr_h is not None else qo_indptr)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    qd = q_dtype if q_dtype is not None else (q_p.dtype if q_p is not None else q_d.dtype)
    od = o_dtype if o_dtype is not None else (o_p.dtype if o_p is not None else o_d.dtype)
    hq = num_qo_heads if num_qo_heads is not None else (q_p.shape[1] if q_p is not None else q_d.shape[1])
    st = lib().fi_batch_pod_paged(
        _ptr(q_p), _ptr(qo_indptr), qh.data_ptr(), int(batch_p if batch_p is not None else qh.numel() - 1),
        ctypes.byref(kv_p), 1 if causal else 0, _ptr(o_p), _ptr(lse_p), _ptr(q_d),
        int(batch_d if batch_d is not None else q_d.shape[0]), ctypes.byref(kv_d), _ptr(o_d), _ptr(lse_d), _dt(qd),
        _dt(od), int(hq), float(sm_scale), _ptr(workspace), int(workspace_bytes), _stream(stream, q_p, q_d, o_p, o_d))
    check(st)
    return o_p, o_d


def fi_batch_prefill_paged_fp8q(q, qo_indptr, kv: PagedKV, o, *, q_dtype, o_dtype=None, q_scale=1.0, causal=True,
                                pv_fp8=False, lse=None, sm_scale=0.0, qo_indptr_h=None, batch=None, num_qo_heads=None,
                                stream=None):
    """q [total_q, H_qo, D] fp8 codes (a float8 tensor, or uint8 with q_dtype
    naming the format); o [total_q, H_qo, D] float16 or bfloat16."""
    qh = _host_i32(qo_indptr_h if qo_indptr_h is not None else qo_indptr)
    st = lib().fi_batch_prefill_paged_fp8q(
        _ptr(q), _dt(q_dtype), float(q_scale), _ptr(qo_indptr), qh.data_ptr(),
        int(batch if batch is not None else qh.numel() - 1), int(num_qo_heads if num_qo_heads is not None else q.shape[1]),
        ctypes.byref(kv), 1 if causal else 0, 1 if pv_fp8 else 0, _ptr(o),
        _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse), float(sm_scale), _stream(stream, q, o))
    check(st)
    return o


def make_ragged_kv(k, v, indptr, *, k_scale=1.0, v_scale=1.0, kv_dtype=None, k_dtype=None, v_dtype=None,
                   indptr_h=None):
    """Describe a ragged K/V: k and v are [num_tokens, H_kv, head_dim] tensors
    with a contiguous last dimension, request i owning rows indptr[i] ..
    indptr[i+1]-1; raw fp8 may be passed as uint8 with kv_dtype naming the
    format.  Returns (struct, keepalive); keepalive holds every tensor the
    struct points at."""
    if tuple(k.stride()) != tuple(v.stride()) or k.shape != v.shape:
        raise FiValueError(2, "k and v must have the same shape and strides")
    kd = k_dtype if k_dtype is not None else (kv_dtype if kv_dtype is not None else k.dtype)
    vd = v_dtype if v_dtype is not None else (kv_dtype if kv_dtype is not None else v.dtype)
    ih = _host_i32(indptr_h if indptr_h is not None else indptr)
    s = RaggedKV()
    s.k, s.v = _ptr(k), _ptr(v)
    s.k_dtype, s.v_dtype = _dt(kd), _dt(vd)
    s.stride_token, s.stride_head = k.stride(0), k.stride(1)
    s.num_tokens, s.num_kv_heads, s.head_dim = int(k.shape[0]), int(k.shape[1]), int(k.shape[2])
    s.indptr, s.indptr_h = _ptr(indptr), ih.data_ptr()
    s.k_scale, s.v_scale = float(k_scale), float(v_scale)
    return s, (ih, k, v, indptr)


def fi_batch_prefill_ragged(q, qo_indptr, kv: RaggedKV, o, *, causal=True, q_dtype=None, o_dtype=None, lse=None,
                            sm_scale=0.0, qo_indptr_h=None, batch=None, num_qo_heads=None, stream=None):
    """q and o [total_q, H_qo, D]; qo_indptr [batch+1] int32 (device)."""
    qh = _host_i32(qo_indptr_h if qo_indptr_h is not None else qo_indptr)
    st = lib().fi_batch_prefill_ragged(
        _ptr(q), _dt(q_dtype if q_dtype is not None else q.dtype), _ptr(qo_indptr), qh.data_ptr(),
        int(batch if batch is not None else qh.numel() - 1), int(num_qo_heads if num_qo_heads is not None else q.shape[1]),
        ctypes.byref(kv), 1 if causal else 0, _ptr(o), _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse),
        float(sm_scale), _stream(stream, q, o))
    check(st)
    return o


def fi_batch_prefill_ragged_fp8q(q, qo_indptr, kv: RaggedKV, o, *, q_dtype, o_dtype=None, q_scale=1.0, causal=True,
                                 pv_fp8=False, lse=None, sm_scale=0.0, qo_indptr_h=None, batch=None, num_qo_heads=None,
                                 stream=None):
    """q [total_q, H_qo, D] fp8 codes (a float8 tensor, or uint8 with q_dtype
    naming the format); o [total_q, H_qo, D] float16 or bfloat16."""
    qh = _host_i32(qo_indptr_h if qo_indptr_h is not None else qo_indptr)
    st = lib().fi_batch_prefill_ragged_fp8q(
        _ptr(q), _dt(q_dtype), float(q_scale), _ptr(qo_indptr), qh.data_ptr(),
        int(batch if batch is not None else qh.numel() - 1), int(num_qo_heads if num_qo_heads is not None else q.shape[1]),
        ctypes.byref(kv), 1 if causal else 0, 1 if pv_fp8 else 0, _ptr(o),
        _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse), float(sm_scale), _stream(stream, q, o))
    check(st)
    return o


def fi_single_prefill_fp8q(q, k, v, o, *, q_dtype, q_scale=1.0, causal=True, pv_fp8=False, k_scale=1.0, v_scale=1.0,
                           kv_dtype=None, k_dtype=None, v_dtype=None, o_dtype=None, lse=None, sm_scale=0.0,
                           stream=None):
    """q [qo_len, H_qo, D] fp8 codes; k and v contiguous [kv_len, H_kv, D] fp8
    codes; o [qo_len, H_qo, D] float16 or bfloat16."""
    kd = k_dtype if k_dtype is not None else (kv_dtype if kv_dtype is not None else k.dtype)
    vd = v_dtype if v_dtype is not None else (kv_dtype if kv_dtype is not None else v.dtype)
    st = lib().fi_single_prefill_fp8q(
        _ptr(q), _dt(q_dtype), float(q_scale), int(q.shape[0]), _ptr(k), _ptr(v), _dt(kd), _dt(vd), int(k.shape[0]),
        int(q.shape[1]), int(k.shape[1]), int(k.shape[2]), 1 if causal else 0, 1 if pv_fp8 else 0, float(k_scale),
        float(v_scale), _ptr(o), _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse), float(sm_scale),
        _stream(stream, q, o))
    check(st)
    return o


def fi_single_prefill(q, k, v, o, *, causal=True, k_scale=1.0, v_scale=1.0, q_dtype=None, kv_dtype=None,
                      k_dtype=None, v_dtype=None, o_dtype=None, lse=None, sm_scale=0.0, stream=None):
    """q and o [qo_len, H_qo, D]; k and v contiguous [kv_len, H_kv, D]."""
    kd = k_dtype if k_dtype is not None else (kv_dtype if kv_dtype is not None else k.dtype)
    vd = v_dtype if v_dtype is not None else (kv_dtype if kv_dtype is not None else v.dtype)
    st = lib().fi_single_prefill(
        _ptr(q), _dt(q_dtype if q_dtype is not None else q.dtype), int(q.shape[0]), _ptr(k), _ptr(v), _dt(kd), _dt(vd),
        int(k.shape[0]), int(q.shape[1]), int(k.shape[1]), int(k.shape[2]), 1 if causal else 0, float(k_scale),
        float(v_scale), _ptr(o), _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse), float(sm_scale),
        _stream(stream, q, o))
    check(st)
    return o


def fi_single_decode(q, k, v, o, *, k_scale=1.0, v_scale=1.0, q_dtype=None, kv_dtype=None, k_dtype=None,
                     v_dtype=None, o_dtype=None, lse=None, sm_scale=0.0, workspace=None, workspace_bytes=None,
                     stream=None):
    """q and o [H_qo, D]; k and v contiguous [kv_len, H_kv, D]."""
    kd = k_dtype if k_dtype is not None else (kv_dtype if kv_dtype is not None else k.dtype)
    vd = v_dtype if v_dtype is not None else (kv_dtype if kv_dtype is not None else v.dtype)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    st = lib().fi_single_decode(
        _ptr(q), _dt(q_dtype if q_dtype is not None else q.dtype), _ptr(k), _ptr(v), _dt(kd), _dt(vd),
        int(k.shape[0]), int(q.shape[0]), int(k.shape[1]), int(k.shape[2]), float(k_scale), float(v_scale), _ptr(o),
        _dt(o_dtype if o_dtype is not None else o.dtype), _ptr(lse), float(sm_scale), _ptr(workspace),
        int(workspace_bytes), _stream(stream, q, o))
    check(st)
    return o


def fi_fp8_widen(codes, src_dtype, out, dst_dtype=None, stream=None):
    """codes uint8 [n] -> out 2-byte [n] (device tensors)."""
    st = lib().fi_fp8_widen(_ptr(codes), int(codes.numel()), _dt(src_dtype),
                            _dt(dst_dtype if dst_dtype is not None else out.dtype), _ptr(out), _stream(stream, codes, out))
    check(st)
    return out
