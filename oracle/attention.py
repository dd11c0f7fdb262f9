"""Plain fp64 CPU definition of batched attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does, and it
shares no code, table or constant generator with the HIP library.

What is computed, and where the pages state it:
  * The paged cache (indptr / indices / last_page_len, a fixed page size, a
    request's last page partly filled) and GQA head grouping: "Enable Hopper
    FA3 FP8 attention in decode.py" (flashinfer PR #2148), Walkthrough and
    review comments on plan()/run(); "fp8 KV cache in the in-tree prefill
    kernel" (AMD-Ecosystem/flashinfer PR #368), Summary and Benchmark results
    (GQA 32/8, head_dim 128, page 16).
  * fp8 K/V with per-tensor k_scale / v_scale: real K = stored value * k_scale,
    real V = stored value * v_scale (PR #368, Test plan, the k_scale/v_scale
    item; PR #2148, review comments on the v_scale multiply).
  * An fp8 query carries a per-tensor q_scale: real q = stored value *
    q_scale (PR #2148, review comments: q_scale folded into sm_scale for the
    first product).
  * The output has q's shape with V's head_dim (PR #2148, Nitpick comments).
  * Causal prefill (PR #368, Benchmark results).  Where the pages are silent
    (mask alignment, default softmax scale, log base of the LSE, empty
    requests) this module takes the plainest reading:
      - the causal mask is aligned to the end of the KV sequence: query row r of
        a request with qo_len queries and kv_len keys sees key t iff
        t <= r + kv_len - qo_len;
      - sm_scale defaults to 1/sqrt(head_dim);
      - lse is the natural-log log-sum-exp of the scaled logits;
      - a row with no visible key has o = 0 and lse = -inf (the identity of the
        state merge); a NaN stored in K or V is not an empty row, it
        propagates through the arithmetic as IEEE floats do, to the rows
        that see its key and to no other.
  * The split-KV state merge (PR #2148, the fixed_split_size /
    disable_split_kv plan arguments): L = ln sum_c exp(lse_c),
    o = sum_c exp(lse_c - L) o_c.

Everything is float64.  The softmax is the exact two-pass form: row max, then
exp and sum.  Each request and kv head is done with the group's query rows
stacked into one matrix product (a library matmul is one step of the
definition, nothing more).
"""
from __future__ import annotations

import math

import numpy as np

from .fp8 import fp8_table

TWO_BYTE = ("f16", "bf16")
FP8 = ("e4m3", "e5m2", "e4m3fnuz", "e5m2fnuz")


# --------------------------------------------------------------------------
# element decoding
# --------------------------------------------------------------------------
def decode_2byte(bits: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 bit patterns of an IEEE binary16 or a bfloat16 -> exact float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # bfloat16 is the upper half of an IEEE binary32
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"not a 2-byte float dtype: {dtype}")


def decode_elements(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored KV / q elements -> float64 values (no scaling)."""
    if dtype in FP8:
        return fp8_table(dtype)[np.asarray(raw, dtype=np.uint8)]
    return decode_2byte(raw, dtype)


# --------------------------------------------------------------------------
# paged cache walk
# --------------------------------------------------------------------------
def kv_len_of(indptr, last_page_len, page_size: int, i: int) -> int:
    npages = int(indptr[i + 1]) - int(indptr[i])
    if npages == 0:
        return 0
    return (npages - 1) * page_size + int(last_page_len[i])


def gather_request(pool: np.ndarray, indptr, indices, last_page_len, page_size: int, i: int) -> np.ndarray:
    """Logical token t of request i lives on page indices[indptr[i] + t // page_size]
    in slot t % page_size.  pool is [num_pages, page_size, H_kv, d] (raw elements).
    Returns [kv_len, H_kv, d] raw elements in token order."""
    n = kv_len_of(indptr, last_page_len, page_size, i)
    if n == 0:
        return pool[:0, 0]
    t = np.arange(n)
    pages = np.asarray(indices)[int(indptr[i]) + t // page_size]
    slots = t % page_size
    return pool[pages, slots]


# --------------------------------------------------------------------------
# the attention definition
# --------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool, sm_scale: float):
    """q [n_q, H_qo, d], k and v [n_kv, H_kv, d], all float64 real values.

    Query head h reads kv head h // (H_qo // H_kv).  Row r sees key t iff
    t < n_kv and, when causal, t <= r + n_kv - n_q.

    Returns o [n_q, H_qo, d] and lse [n_q, H_qo] (natural log), float64."""
    n_q, h_qo, d = q.shape
    n_kv, h_kv, _ = k.shape
    assert h_qo % h_kv == 0
    group = h_qo // h_kv
    o = np.zeros((n_q, h_qo, d), dtype=np.float64)
    lse = np.full((n_q, h_qo), -np.inf, dtype=np.float64)
    if n_q == 0 or n_kv == 0:
        return o, lse
    rows = np.arange(n_q)[:, None]
    cols = np.arange(n_kv)[None, :]
    if causal:
        allowed = cols <= rows + (n_kv - n_q)  # [n_q, n_kv]
    else:
        allowed = np.ones((n_q, n_kv), dtype=bool)
    for g in range(h_kv):
        kg = k[:, g, :]  # [n_kv, d]
        vg = v[:, g, :]
        qg = q[:, g * group:(g + 1) * group, :]  # [n_q, group, d]
        s = (qg.reshape(n_q * group, d) @ kg.T) * sm_scale  # [n_q*group, n_kv]
        s = s.reshape(n_q, group, n_kv)
        mask = np.broadcast_to(allowed[:, None, :], s.shape)
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=-1, keepdims=True)  # -inf on empty rows; NaN if a visible logit is NaN
        # a row is empty when the mask leaves it no key; a NaN stored in K or V
        # is not an empty row: it propagates through exp and the sums
        has = np.broadcast_to(allowed.any(axis=-1)[:, None, None], m.shape)
        m_safe = np.where(has, m, 0.0)
        p = np.exp(s - m_safe)  # exp(-inf) = 0 on masked entries
        denom = p.sum(axis=-1, keepdims=True)
        w = np.where(has, p / np.where(has, denom, 1.0), 0.0)
        # a key the mask hides contributes nothing to a row, also when its
        # stored V is not finite (a zero weight times NaN or inf would reach
        # the row): the product runs over finite V, and each non-finite
        # element is added to the rows that see its key alone
        vfin = np.isfinite(vg)
        og = (w.reshape(n_q * group, n_kv) @ np.where(vfin, vg, 0.0)).reshape(n_q, group, d)
        for t, c in zip(*np.nonzero(~vfin)):
            sees = allowed[:, t]
            og[sees, :, c] += w[sees, :, t] * vg[t, c]
        o[:, g * group:(g + 1) * group, :] = og
        lse[:, g * group:(g + 1) * group] = np.where(has[..., 0], m[..., 0] + np.log(np.where(has[..., 0], denom[..., 0], 1.0)), -np.inf)
    return o, lse


def default_sm_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def _resolve_scale(sm_scale, head_dim):
    return default_sm_scale(head_dim) if (sm_scale is None or sm_scale <= 0) else float(sm_scale)


# --------------------------------------------------------------------------
# batched entry points over a paged cache, on raw stored elements
# --------------------------------------------------------------------------
def paged_kv_values(w: dict, i: int):
    """Real-valued K and V (scales applied) of request i, [kv_len, H_kv, d]."""
    k_raw = gather_request(w["k_pool"], w["indptr"], w["indices"], w["last_page_len"], w["page_size"], i)
    v_raw = gather_request(w["v_pool"], w["indptr"], w["indices"], w["last_page_len"], w["page_size"], i)
    k = decode_elements(k_raw, w["kv_dtype"]) * float(w["k_scale"])
    v = decode_elements(v_raw, w["kv_dtype"]) * float(w["v_scale"])
    return k, v


def query_values(w: dict) -> np.ndarray:
    """Real-valued queries [tokens, H_qo, d]: the stored elements times the
    per-tensor q_scale of an fp8 query (1 for a 2-byte query).  The scale
    multiplies q exactly as k_scale multiplies K ("Enable Hopper FA3 FP8
    attention in decode.py", flashinfer PR #2148, review comments: q_scale
    folded into sm_scale for the first product)."""
    return decode_elements(w["q"], w["q_dtype"]) * float(w.get("q_scale", 1.0))


def batch_attention(w: dict, *, causal: bool, sm_scale=None, requests=None):
    """Attention for every request of a workload dict (see workloads.gen).
    Decode is qo_len = 1 per request (qo_indptr = arange(B+1)).

    Returns o [tokens, H_qo, d] and lse [tokens, H_qo] in float64."""
    q_all = query_values(w)
    d = q_all.shape[-1]
    scale = _resolve_scale(sm_scale, d)
    qo_indptr = w["qo_indptr"]
    o = np.zeros_like(q_all)
    lse = np.full(q_all.shape[:2], -np.inf)
    reqs = range(len(qo_indptr) - 1) if requests is None else requests
    for i in reqs:
        a, b = int(qo_indptr[i]), int(qo_indptr[i + 1])
        k, v = paged_kv_values(w, i)
        o[a:b], lse[a:b] = attention(q_all[a:b], k, v, causal=causal, sm_scale=scale)
    return o, lse


def batch_decode(w: dict, sm_scale=None, requests=None):
    return batch_attention(w, causal=False, sm_scale=sm_scale, requests=requests)


def batch_prefill(w: dict, causal: bool = True, sm_scale=None, requests=None):
    return batch_attention(w, causal=causal, sm_scale=sm_scale, requests=requests)


def single_decode(q_raw, q_dtype, k_raw, v_raw, kv_dtype, k_scale, v_scale, sm_scale=None):
    """q [H_qo, d]; contiguous k, v [kv_len, H_kv, d] raw elements."""
    q = decode_elements(q_raw, q_dtype)[None]
    k = decode_elements(k_raw, kv_dtype) * float(k_scale)
    v = decode_elements(v_raw, kv_dtype) * float(v_scale)
    o, lse = attention(q, k, v, causal=False, sm_scale=_resolve_scale(sm_scale, q.shape[-1]))
    return o[0], lse[0]


def attention_rows(w: dict, token_ids, head_ids, *, causal: bool, sm_scale=None):
    """Outputs for a sample of (query token, q head) pairs, each computed on its
    own: for checks at sizes where the full oracle would take too long."""
    q_all = query_values(w)
    d = q_all.shape[-1]
    scale = _resolve_scale(sm_scale, d)
    qo_indptr = np.asarray(w["qo_indptr"])
    h_qo = q_all.shape[1]
    h_kv = w["k_pool"].shape[2]
    group = h_qo // h_kv
    out_o = np.zeros((len(token_ids), d))
    out_l = np.zeros(len(token_ids))
    cache = {}
    for n, (tok, h) in enumerate(zip(token_ids, head_ids)):
        i = int(np.searchsorted(qo_indptr, tok, side="right") - 1)
        if i not in cache:
            cache = {i: paged_kv_values(w, i)}
        k, v = cache[i]
        g = h // group
        r = tok - int(qo_indptr[i])
        n_q = int(qo_indptr[i + 1]) - int(qo_indptr[i])
        qq = q_all[tok:tok + 1, h:h + 1]
        o1, l1 = attention_causal_row(qq[0, 0], k[:, g], v[:, g], r, n_q, causal, scale)
        out_o[n], out_l[n] = o1, l1
    return out_o, out_l


def attention_causal_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, r: int, n_q: int, causal: bool, sm_scale: float):
    """One query row against one kv head: q [d], k and v [n_kv, d]."""
    n_kv = k.shape[0]
    lim = n_kv if not causal else min(n_kv, r + n_kv - n_q + 1)
    if lim <= 0:
        return np.zeros(q.shape[-1]), -np.inf
    s = (k[:lim] @ q) * sm_scale
    m = s.max()
    p = np.exp(s - m)
    den = p.sum()
    return (p / den) @ v[:lim], m + math.log(den)


# --------------------------------------------------------------------------
# split-KV state merge
# --------------------------------------------------------------------------
def merge_states(o_parts: np.ndarray, lse_parts: np.ndarray):
    """o_parts [C, ..., d], lse_parts [C, ...] (natural log).  Chunks with
    lse = -inf carry no weight; if every chunk is empty the result is o = 0,
    lse = -inf."""
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    has = ~np.all(np.isneginf(lse_parts), axis=0)  # a NaN state propagates
    m_safe = np.where(has, m, 0.0)
    wts = np.exp(lse_parts - m_safe)  # [C, ...]
    tot = wts.sum(axis=0)
    L = np.where(has, m_safe + np.log(np.where(has, tot, 1.0)), -np.inf)
    coef = np.where(has, wts / np.where(has, tot, 1.0), 0.0)
    o = (coef[..., None] * o_parts).sum(axis=0)
    return o, L
