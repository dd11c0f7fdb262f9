"""Helpers for the GPU parity tests: move a seeded workload to the device, call
the library through its C ABI binding, and compare with the oracle.

Tolerances (max |GPU - oracle| over all elements, oracle in float64): 1e-2 for
a float16 output, 2e-2 for bfloat16; the log-sum-exp within 1e-3 absolute.
A non-finite value anywhere fails.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

from attention_paged_fp8_amd import fi

T2 = {"f16": torch.float16, "bf16": torch.bfloat16}
O_TOL = {"f16": 1e-2, "bf16": 2e-2}
LSE_TOL = 1e-3


def say(*a):
    """Name the case on stdout before a GPU step."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev_2byte(bits: np.ndarray, dtype: str, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(T2[dtype]).to(device)


def dev_pool(pool: np.ndarray, kvd: str, device) -> torch.Tensor:
    if kvd in T2:
        return dev_2byte(pool, kvd, device)
    return torch.from_numpy(np.ascontiguousarray(pool)).to(device)  # raw uint8 codes


def upload(w: dict, device) -> dict:
    d = dict(
        q=dev_pool(w["q"], w["q_dtype"], device),  # fp8 queries stay raw codes
        k=dev_pool(w["k_pool"], w["kv_dtype"], device),
        v=dev_pool(w["v_pool"], w["kv_dtype"], device),
        indptr=torch.from_numpy(w["indptr"]).to(device),
        indices=torch.from_numpy(np.ascontiguousarray(w["indices"], dtype=np.int32)).to(device),
        lpl=torch.from_numpy(w["last_page_len"]).to(device),
        qo_indptr=torch.from_numpy(w["qo_indptr"]).to(device),
    )
    return d


def paged_kv(w: dict, d: dict, k=None, v=None, kv_dtype=None, k_scale=None, v_scale=None):
    return fi.make_paged_kv(
        d["k"] if k is None else k, d["v"] if v is None else v, d["indptr"], d["indices"], d["lpl"],
        k_scale=w["k_scale"] if k_scale is None else k_scale, v_scale=w["v_scale"] if v_scale is None else v_scale,
        kv_dtype=kv_dtype or w["kv_dtype"], indptr_h=w["indptr"], last_page_len_h=w["last_page_len"])


def workspace_for(w: dict, device) -> torch.Tensor:
    n = fi.fi_decode_workspace_bytes(len(w["kv_lens"]), w["num_qo_heads"], w["head_dim"],
                                     int(max(1, w["kv_lens"].max())))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def run_decode(w: dict, d: dict, *, o_dtype=None, workspace=True, sm_scale=0.0, kv=None, split=None):
    """Returns (o as float64 numpy, lse numpy, o tensor)."""
    od = o_dtype or w["o_dtype"]
    B = len(w["kv_lens"])
    o = torch.full((B, w["num_qo_heads"], w["head_dim"]), float("nan"), dtype=T2[od], device=d["q"].device)
    lse = torch.full((B, w["num_qo_heads"]), float("nan"), dtype=torch.float32, device=d["q"].device)
    ws = workspace_for(w, d["q"].device) if workspace else None
    if kv is None:
        kv, keep = paged_kv(w, d)
    old = os.environ.get("FI_SPLIT_KV")
    try:
        if split is not None:
            os.environ["FI_SPLIT_KV"] = str(split)
        fi.fi_batch_decode_paged(d["q"], kv, o, lse=lse, sm_scale=sm_scale, workspace=ws)
    finally:
        if split is not None:
            if old is None:
                os.environ.pop("FI_SPLIT_KV", None)
            else:
                os.environ["FI_SPLIT_KV"] = old
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), o


def run_prefill(w: dict, d: dict, *, causal=True, o_dtype=None, sm_scale=0.0, kv=None):
    od = o_dtype or w["o_dtype"]
    T = int(w["qo_indptr"][-1])
    o = torch.full((T, w["num_qo_heads"], w["head_dim"]), float("nan"), dtype=T2[od], device=d["q"].device)
    lse = torch.full((T, w["num_qo_heads"]), float("nan"), dtype=torch.float32, device=d["q"].device)
    if kv is None:
        kv, keep = paged_kv(w, d)
    fi.fi_batch_prefill_paged(d["q"], d["qo_indptr"], kv, o, causal=causal, lse=lse, sm_scale=sm_scale,
                              qo_indptr_h=w["qo_indptr"])
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), o


def assert_parity(o, lse, o_ref, lse_ref, o_dtype: str, what: str = ""):
    assert np.all(np.isfinite(o)), f"{what}: non-finite output ({np.sum(~np.isfinite(o))} elements)"
    err = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    assert err <= O_TOL[o_dtype], f"{what}: max |o - oracle| = {err:.3e} > {O_TOL[o_dtype]}"
    if lse is not None:
        both_inf = np.isneginf(lse) & np.isneginf(lse_ref)
        fin = ~both_inf
        assert np.all(np.isfinite(lse[fin])) and np.all(np.isfinite(lse_ref[fin])), f"{what}: lse -inf mismatch"
        lerr = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
        assert lerr <= LSE_TOL, f"{what}: max |lse - oracle| = {lerr:.3e} > {LSE_TOL}"
    return err


def assert_parity_nan(o, lse, o_ref, lse_ref, o_dtype: str, what: str = ""):
    """Parity where the oracle holds NaNs (a NaN code in the cache): the GPU
    output is NaN at exactly the oracle's NaN elements of o and lse, and every
    other element is held to the usual tolerance."""
    o_nan, l_nan = np.isnan(o_ref), np.isnan(lse_ref)
    assert o_nan.any(), f"{what}: the case plants no NaN the oracle sees"
    assert np.array_equal(np.isnan(o), o_nan), \
        f"{what}: NaN outputs differ from the oracle's ({np.sum(np.isnan(o) != o_nan)} elements)"
    assert np.array_equal(np.isnan(lse), l_nan), \
        f"{what}: NaN lse differ from the oracle's ({np.sum(np.isnan(lse) != l_nan)} rows)"
    return assert_parity(np.where(o_nan, 0.0, o), np.where(l_nan, 0.0, lse), np.where(o_nan, 0.0, o_ref),
                         np.where(l_nan, 0.0, lse_ref), o_dtype, what)


def plant_codes(w: dict, i: int, spots) -> None:
    """Write stored codes into request i's K or V elements: spots holds
    (pool name "k_pool" or "v_pool", token, kv head, dimension, code)."""
    ps = w["page_size"]
    for pool, t, g, c, code in spots:
        w[pool][w["indices"][w["indptr"][i] + t // ps], t % ps, g, c] = code
