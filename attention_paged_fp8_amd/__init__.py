"""Paged fp8-KV attention (decode and causal prefill) for MI355X / gfx950.

The computation lives in libfi.so (HIP kernels behind the C ABI of
include/fi.h); ``attention_paged_fp8_amd.fi`` is its Python binding.
Build the library with ``python -m attention_paged_fp8_amd.build``.
"""
from .fi import (  # noqa: F401
    FiError, FiRuntimeError, FiValueError, PagedKV, fi_batch_decode_paged, fi_batch_prefill_paged,
    fi_decode_workspace_bytes, fi_fp8_widen, fi_single_decode, lib, make_paged_kv,
)
