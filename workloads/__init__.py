"""Seeded synthetic inputs for paged fp8-KV attention.

This module is shared by the tests, the smoke check and the benchmark.  It
draws random numbers and encodes them into the stored formats with library
casts (torch's float16 / bfloat16 / float8 conversions, round to nearest even);
it holds none of the attention arithmetic and imports neither the oracle nor
the library.

Shapes follow the workloads of the pages: GQA 32 q heads / 8 kv heads,
head_dim 128, page 16 ("fp8 KV cache in the in-tree prefill kernel",
AMD-Ecosystem/flashinfer PR #368, Benchmark results), plus the workloads
this library is measured on (``WORKLOADS``, by name).  Values are N(0, 1): the pages use
model activations but provide none, so standard normals stand in.

Draw order for one workload (numpy default_rng(seed)):
  1. lengths: kv lengths (decode) or qo lengths then prefix lengths (prefill),
     each ``integers(lo, hi + 1)``;
  2. the page order: ``arange`` when pages are contiguous, else a permutation of
     the page pool (the pool holds exactly the pages needed, plus
     ``extra_pages`` unreferenced ones);
  3. q, standard normal float32, cast to q's dtype (an fp8 query is scaled
     per tensor like K and V below: q_scale = amax / max finite);
  4. K, then V: standard normal float32 over the whole pool.  fp8: per-tensor
     scale = amax over valid slots / max finite (448 for e4m3, 57344 for e5m2);
     x / scale clamped to +-max finite, cast round-to-nearest-even.  2-byte:
     cast directly, scale 1.
  5. slots past last_page_len, and unreferenced pages, are poisoned with a NaN
     encoding (0x7F for OCP fp8, 0x80 for fnuz fp8, the canonical quiet NaN for
     2-byte types), so an out-of-range read shows up as a non-finite output.
"""
from __future__ import annotations

import numpy as np
import torch

FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0, "e4m3fnuz": 240.0, "e5m2fnuz": 57344.0}
_TORCH = {
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "e4m3": torch.float8_e4m3fn,
    "e5m2": torch.float8_e5m2,
    "e4m3fnuz": torch.float8_e4m3fnuz,
    "e5m2fnuz": torch.float8_e5m2fnuz,
}
NAN_BITS = {"e4m3": 0x7F, "e5m2": 0x7F, "e4m3fnuz": 0x80, "e5m2fnuz": 0x80, "f16": 0x7E00, "bf16": 0x7FC0}
ELEM_BYTES = {"f16": 2, "bf16": 2, "e4m3": 1, "e5m2": 1, "e4m3fnuz": 1, "e5m2fnuz": 1}

# The measured workloads, by name, each with a fixed seed.  The dtype-comparison
# decode reuses the batch-decode seed, so its three legs have the batch-decode
# workload's lengths, page permutation and draws (cast to f16 and to its KV type).
WORKLOADS = {
    "single_decode": dict(seed=1, name="single_decode_kv64_h4-4_d64_page16_e4m3_f16", kind="single_decode", batch=1,
            kv=(64, 64), hq=4, hkv=4, d=64, page=16, q="f16", kvd="e4m3", o="f16", contiguous=True),
    "batch_decode": dict(seed=2, name="batch_decode_b64_kv512-4096_h32-8_d128_page16_e4m3_bf16", kind="decode", batch=64,
            kv=(512, 4096), hq=32, hkv=8, d=128, page=16, q="bf16", kvd="e4m3", o="bf16", contiguous=False),
    "causal_prefill": dict(seed=3, name="causal_prefill_b16_qo256-1024_prefix0-2048_h32-8_d128_page16_e4m3_f16", kind="prefill",
            batch=16, qo=(256, 1024), prefix=(0, 2048), hq=32, hkv=8, d=128, page=16, q="f16", kvd="e4m3",
            o="f16", contiguous=False),
    "long_context_decode": dict(seed=4, name="splitkv_decode_b8_kv32768-131072_h64-8_d128_page64_e5m2_bf16", kind="decode", batch=8,
            kv=(32768, 131072), hq=64, hkv=8, d=128, page=64, q="bf16", kvd="e5m2", o="bf16", contiguous=False),
    "dtype_decode": dict(seed=2, name="dtype_decode_b64_kv512-4096_h32-8_d128_page16_f16q", kind="decode", batch=64,
            kv=(512, 4096), hq=32, hkv=8, d=128, page=16, q="f16", kvd=("f16", "bf16", "e4m3"), o="f16",
            contiguous=False),
}


def cast_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> stored bit patterns (uint16 for 2-byte, uint8 for fp8)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(_TORCH[dtype])
    if dtype in ("f16", "bf16"):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


def _encode_pool(x: np.ndarray, dtype: str, valid: np.ndarray):
    """Encode a float32 pool [P, page, H, d]; valid is a [P, page] bool mask."""
    P = x.shape[0]
    step = max(1, (1 << 25) // max(1, int(np.prod(x.shape[1:]))))  # rows per block (an empty pool has none)
    xt = torch.from_numpy(x)
    vt = torch.from_numpy(valid)
    if dtype in FP8_MAX:
        amax = 0.0
        for a in range(0, P, step):
            blk = xt[a:a + step].abs().amax(dim=(2, 3))  # [n, page]
            blk = torch.where(vt[a:a + step], blk, torch.zeros_like(blk))
            amax = max(amax, float(blk.max()) if blk.numel() else 0.0)
        scale = amax / FP8_MAX[dtype] if amax > 0 else 1.0
        m = FP8_MAX[dtype]
        out = torch.empty(x.shape, dtype=torch.uint8)
        for a in range(0, P, step):
            y = (xt[a:a + step] / np.float32(scale)).clamp_(-m, m)
            out[a:a + step] = y.to(_TORCH[dtype]).view(torch.uint8)
        return out.numpy(), float(scale)
    out = torch.empty(x.shape, dtype=torch.int16)
    for a in range(0, P, step):
        out[a:a + step] = xt[a:a + step].to(_TORCH[dtype]).view(torch.int16)
    return out.numpy().view(np.uint16), 1.0


def make_paged(seed: int, *, kv_lens=None, qo_lens=None, prefix_lens=None, hq: int, hkv: int, d: int,
               page: int, q: str, kvd: str, o: str | None = None, contiguous: bool = False,
               extra_pages: int = 0, kv_range=None, qo_range=None, prefix_range=None, batch=None,
               poison: bool = True) -> dict:
    """Build one workload.  Either give the lengths directly or give ranges plus
    a batch size (lengths are then drawn first, as described above).

    Decode: ``kv_lens`` (qo_len = 1 per request).  Prefill: ``qo_lens`` and
    ``prefix_lens`` (kv_len = qo_len + prefix_len), or ``qo_lens`` and
    ``kv_lens`` directly."""
    rng = np.random.default_rng(seed)
    if kv_range is not None:
        kv_lens = rng.integers(kv_range[0], kv_range[1] + 1, size=batch)
    if qo_range is not None:
        qo_lens = rng.integers(qo_range[0], qo_range[1] + 1, size=batch)
        prefix_lens = rng.integers(prefix_range[0], prefix_range[1] + 1, size=batch)
    if qo_lens is None:
        kv_lens = np.asarray(kv_lens, dtype=np.int64)
        qo_lens = np.ones_like(kv_lens)
    else:
        qo_lens = np.asarray(qo_lens, dtype=np.int64)
        if kv_lens is not None and prefix_lens is None:
            kv_lens = np.asarray(kv_lens, dtype=np.int64)  # explicit, may be shorter than qo_lens
        else:
            prefix_lens = np.zeros_like(qo_lens) if prefix_lens is None else np.asarray(prefix_lens, dtype=np.int64)
            kv_lens = qo_lens + prefix_lens
    B = len(kv_lens)
    npages = (kv_lens + page - 1) // page
    indptr = np.zeros(B + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(npages)
    P_used = int(indptr[-1])
    P = P_used + extra_pages
    last_page_len = np.where(kv_lens > 0, kv_lens - (npages - 1) * page, 0).astype(np.int32)
    # convention for empty requests: no pages; last_page_len is ignored but kept in [1, page]
    last_page_len = np.where(npages == 0, 1, last_page_len).astype(np.int32)
    order = np.arange(P, dtype=np.int64) if contiguous else rng.permutation(P)
    indices = order[:P_used].astype(np.int32)

    qo_indptr = np.zeros(B + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    q32 = rng.standard_normal((int(qo_indptr[-1]), hq, d), dtype=np.float32)
    if q in FP8_MAX:  # an fp8 query: per-tensor scale amax / max finite, as for K and V
        q_bits, q_scale = _encode_pool(q32[:, None], q, np.ones((q32.shape[0], 1), dtype=bool))
        q_bits = q_bits[:, 0]
    else:
        q_bits, q_scale = cast_bits(q32, q), 1.0
    del q32

    # valid-slot mask over the pool [P, page]
    valid = np.zeros((P, page), dtype=bool)
    for i in range(B):
        pg = indices[indptr[i]:indptr[i + 1]]
        if len(pg) == 0:
            continue
        valid[pg[:-1], :] = True
        valid[pg[-1], :last_page_len[i]] = True

    pools = {}
    scales = {}
    for name in ("k", "v"):
        x = rng.standard_normal((P, page, hkv, d), dtype=np.float32)
        bits, sc = _encode_pool(x, kvd, valid)
        del x
        if poison:
            bits[~valid] = NAN_BITS[kvd]
        pools[name] = bits
        scales[name] = sc

    return dict(
        seed=seed, q=q_bits, q_dtype=q, q_scale=q_scale, kv_dtype=kvd, o_dtype=o or (q if q in ("f16", "bf16") else "f16"),
        k_pool=pools["k"], v_pool=pools["v"], k_scale=scales["k"], v_scale=scales["v"],
        indptr=indptr, indices=indices, last_page_len=last_page_len, page_size=page,
        qo_indptr=qo_indptr, kv_lens=kv_lens.astype(np.int64), qo_lens=qo_lens.astype(np.int64),
        num_qo_heads=hq, num_kv_heads=hkv, head_dim=d, num_pages=P, valid=valid,
    )


def make_workload(key: str, kvd: str | None = None, q: str | None = None) -> dict:
    """One measured workload by name (``WORKLOADS``); "dtype_decode" takes its
    KV dtype as an argument, one of f16, bf16, e4m3 (default e4m3), and any
    workload may be drawn with another KV dtype.  ``q`` replaces the query
    dtype (e.g. "e4m3": the same draws quantised with a per-tensor scale); the
    name then says so."""
    c = WORKLOADS[key]
    kvd_eff = kvd if kvd is not None else (c["kvd"] if isinstance(c["kvd"], str) else c["kvd"][-1])
    common = dict(hq=c["hq"], hkv=c["hkv"], d=c["d"], page=c["page"], q=q or c["q"], kvd=kvd_eff, o=c["o"],
                  contiguous=c["contiguous"], batch=c["batch"])
    if c["kind"] == "prefill":
        w = make_paged(c["seed"], qo_range=c["qo"], prefix_range=c["prefix"], **common)
    else:
        w = make_paged(c["seed"], kv_range=c["kv"], **common)
    w["workload"] = key
    w["name"] = c["name"] + (f"_q{q}" if q else "")
    w["kind"] = c["kind"]
    return w


def ragged_rows(w: dict, lead: int = 0, tail: int = 0):
    """The K/V of a paged workload laid out contiguously per request
    ("ragged"): request i's tokens, in logical order, become rows indptr[i] ..
    indptr[i+1]-1 of [rows, H_kv, d] arrays of the same stored elements.
    ``lead`` poisoned rows precede the first request and ``tail`` follow the
    last, so a read outside the requests' rows shows up as a non-finite output.

    Returns (k_rows, v_rows, indptr int32 [B+1]).  Data movement only."""
    kv_lens = np.asarray(w["kv_lens"], dtype=np.int64)
    B = len(kv_lens)
    indptr = np.zeros(B + 1, dtype=np.int32)
    indptr[0] = lead
    indptr[1:] = lead + np.cumsum(kv_lens)
    rows = int(indptr[-1]) + tail
    out = []
    for name in ("k_pool", "v_pool"):
        pool = w[name]
        r = np.full((rows,) + pool.shape[2:], NAN_BITS[w["kv_dtype"]], dtype=pool.dtype)
        for i in range(B):
            n = int(kv_lens[i])
            if n == 0:
                continue
            pages = w["indices"][w["indptr"][i]:w["indptr"][i + 1]]
            r[indptr[i]:indptr[i + 1]] = pool[pages].reshape((-1,) + pool.shape[2:])[:n]
        out.append(r)
    return out[0], out[1], indptr
