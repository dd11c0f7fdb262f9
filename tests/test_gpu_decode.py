"""GPU parity tests for decode (batched paged, single) and the fp8 widening,
through the C ABI, against the float64 oracle.

Cases: every fp8 code widened bitwise; the measured single-decode, batch-decode,
long-context and dtype-decode workloads compared element by element at full size; a matrix of small shapes spanning
several 32-token blocks, ragged tails, empty and one-token requests, page
sizes 1..128, head_dim 64 and 128, GQA groups 1..32, all q / KV / o dtype
combinations decode admits (fnuz caches included), forced split-KV; and the invariants: run-to-run
bitwise determinism, bitwise page-permutation invariance, an fp8 run equal
bitwise to a run on the same values pre-widened to q's type (the equivalence
design of "fp8 KV cache in the in-tree prefill kernel", Test plan), the
k_scale fold, constant V, NaN-poisoned padding and unreferenced pages (OCP and
fnuz), a NaN code in the cache reaching exactly the rows that read it, a
non-default (head-major) pool layout; batches past the planner's limits (900
requests: prefix sums scanned on the device; 1100: fixed chunks) and a
page-size-1 request spanning three page-id windows.
"""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from oracle.fp8 import fp8_table
from attention_paged_fp8_amd import fi
from workloads import NAN_BITS, make_paged, make_workload
from gpu_util import (O_TOL, T2, assert_parity, dev_2byte, paged_kv, run_decode, say, upload, workspace_for)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ fp8 codes
@pytest.mark.parametrize("src", ["e4m3", "e5m2", "e4m3fnuz", "e5m2fnuz"])
@pytest.mark.parametrize("dst", ["f16", "bf16"])
def test_fp8_widen_all_codes_bitwise(gpu_device, src, dst):
    say("widen", src, dst)
    codes = torch.arange(256, dtype=torch.uint8, device=gpu_device).repeat(3)  # 768 codes, ragged-free and reused
    codes = torch.cat([codes, codes[:5]])  # a ragged tail of 5
    out = torch.empty(codes.numel(), dtype=T2[dst], device=gpu_device)
    fi.fi_fp8_widen(codes, src, out)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    ref = fp8_table(src)[codes.cpu().numpy()]
    nan = np.isnan(ref)  # OCP e4m3 0x7F/0xFF, e5m2 0x7D-0x7F/0xFD-0xFF, fnuz 0x80
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))  # -0 stays -0


# ------------------------------------------------------------------ the single-decode workload
def test_single_decode_single_and_batch(gpu_device):
    say("single_decode")
    w = make_workload("single_decode")
    d = upload(w, gpu_device)
    o_ref, l_ref = OA.batch_decode(w)
    o_b, l_b, _ = run_decode(w, d)
    assert_parity(o_b, l_b, o_ref, l_ref, "f16", "batch decode")
    # single decode: contiguous K/V [kv_len, H, D] (pages are contiguous in the single-decode workload)
    kv_len = int(w["kv_lens"][0])
    k = d["k"].reshape(-1, w["num_kv_heads"], w["head_dim"])[:kv_len]
    v = d["v"].reshape(-1, w["num_kv_heads"], w["head_dim"])[:kv_len]
    o = torch.full((w["num_qo_heads"], w["head_dim"]), float("nan"), dtype=torch.float16, device=gpu_device)
    lse = torch.empty(w["num_qo_heads"], dtype=torch.float32, device=gpu_device)
    fi.fi_single_decode(d["q"][0], k, v, o, k_scale=w["k_scale"], v_scale=w["v_scale"], kv_dtype="e4m3", lse=lse)
    torch.cuda.synchronize()
    o_s = o.double().cpu().numpy()
    assert_parity(o_s[None], lse.double().cpu().numpy()[None], o_ref, l_ref, "f16", "single decode")
    # the oracle's contiguous single-decode definition agrees, and the two entry points agree bitwise
    o_r2, l_r2 = OA.single_decode(w["q"][0], "f16", w["k_pool"].reshape(-1, 4, 64)[:kv_len],
                                  w["v_pool"].reshape(-1, 4, 64)[:kv_len], "e4m3", w["k_scale"], w["v_scale"])
    assert np.allclose(o_r2, o_ref[0], atol=1e-12)
    assert np.array_equal(o_s, o_b[0])


# ------------------------------------------------------------------ small matrix
SMALL = [
    # (kvd, q, o, page, d, hq, hkv, lens, split)
    ("e4m3", "f16", "f16", 16, 128, 32, 8, (1, 31, 32, 33, 200, 517, 0, 64), None),
    ("e4m3", "bf16", "bf16", 16, 128, 32, 8, (700, 129, 5), "128"),
    ("e5m2", "bf16", "bf16", 64, 128, 64, 8, (1000, 3, 2049), "256"),
    ("e5m2", "f16", "bf16", 4, 64, 8, 2, (77, 300, 1), None),
    ("e4m3", "bf16", "f16", 1, 64, 4, 4, (9, 40, 130), "128"),
    ("e4m3", "f16", "f16", 128, 128, 32, 1, (1500, 260), "128"),   # group 32: two 16-row slices
    ("e4m3", "f16", "f16", 32, 128, 12, 4, (100, 333), None),        # group 3
    ("f16", "f16", "f16", 16, 128, 32, 8, (400, 65, 1), "128"),
    ("bf16", "bf16", "bf16", 16, 64, 16, 2, (257, 31), None),
    ("bf16", "f16", "f16", 16, 128, 32, 8, (600, 90), "128"),        # mixed 2-byte decode
    ("f16", "bf16", "bf16", 8, 128, 8, 8, (300, 12), None),          # mixed the other way
    ("e5m2", "f16", "f16", 2, 128, 16, 16, (55, 1, 0, 1024), "128"),
    # fnuz caches
    ("e4m3fnuz", "f16", "f16", 16, 128, 32, 8, (1, 31, 32, 33, 200, 517, 0, 64), None),
    ("e4m3fnuz", "bf16", "bf16", 16, 128, 32, 8, (700, 129, 5), "128"),
    ("e5m2fnuz", "f16", "bf16", 64, 128, 64, 8, (1000, 3, 2049), "256"),
    ("e5m2fnuz", "bf16", "f16", 4, 64, 8, 2, (77, 300, 1), None),
    ("e4m3fnuz", "bf16", "f16", 4, 64, 8, 2, (77, 300, 1), None),
    ("e4m3fnuz", "f16", "bf16", 32, 64, 16, 16, (55, 1, 0, 1024), "128"),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-q{c[1]}-o{c[2]}-p{c[3]}-d{c[4]}-h{c[5]}x{c[6]}-s{c[8]}" for c in SMALL])
def test_decode_small(gpu_device, case):
    kvd, q, o, page, d, hq, hkv, lens, split = case
    say("decode small", case)
    w = make_paged(11, kv_lens=list(lens), hq=hq, hkv=hkv, d=d, page=page, q=q, kvd=kvd, o=o, extra_pages=3)
    dv = upload(w, gpu_device)
    o_ref, l_ref = OA.batch_decode(w)
    og, lg, _ = run_decode(w, dv, split=split)
    assert_parity(og, lg, o_ref, l_ref, o, str(case))
    # empty requests: o = 0, lse = -inf
    for i, n in enumerate(lens):
        if n == 0:
            assert np.all(og[i] == 0) and np.all(np.isneginf(lg[i]))


# ------------------------------------------------------------------ 8-wave workgroups
LONG = [
    # (kvd, q, o, page, d, hq, hkv, lens)
    ("e4m3", "bf16", "bf16", 16, 128, 32, 8, (1, 31, 700, 2049, 0, 517)),
    ("e5m2", "f16", "f16", 64, 128, 64, 8, (1000, 3, 4097)),
    ("e4m3", "f16", "bf16", 4, 64, 8, 2, (77, 300, 1, 900)),
    ("e5m2", "bf16", "f16", 1, 64, 4, 4, (9, 40, 130)),
    ("e4m3", "f16", "f16", 128, 128, 32, 1, (1500, 260)),   # group 32: two 16-row slices
    ("e4m3", "f16", "f16", 32, 128, 12, 4, (100, 333)),     # group 3
    ("f16", "f16", "f16", 16, 128, 32, 8, (400, 65, 1)),
    ("bf16", "bf16", "bf16", 16, 64, 16, 2, (257, 31)),
    ("e4m3", "bf16", "bf16", 16, 128, 16, 16, (55, 1, 0, 1024)),
]


@pytest.mark.parametrize("case", LONG, ids=[f"{c[0]}-q{c[1]}-o{c[2]}-p{c[3]}-d{c[4]}-h{c[5]}x{c[6]}" for c in LONG])
def test_decode_eight_wave_workgroups(gpu_device, monkeypatch, case):
    """The 8-wave decode kernel (whole rows of up to 8 kv heads per
    workgroup), which the planner picks for long per-workgroup streams,
    forced on small shapes: parity with the oracle."""
    kvd, q, o, page, d, hq, hkv, lens = case
    say("decode 8 waves", case)
    monkeypatch.setenv("FI_DECODE_WAVES", "8")
    w = make_paged(13, kv_lens=list(lens), hq=hq, hkv=hkv, d=d, page=page, q=q, kvd=kvd, o=o, extra_pages=3)
    dv = upload(w, gpu_device)
    o_ref, l_ref = OA.batch_decode(w)
    og, lg, _ = run_decode(w, dv)
    assert_parity(og, lg, o_ref, l_ref, o, str(case))
    for i, n in enumerate(lens):
        if n == 0:
            assert np.all(og[i] == 0) and np.all(np.isneginf(lg[i]))


# ------------------------------------------------------------------ full-size workloads
@pytest.mark.parametrize("wl", ["batch_decode", "long_context_decode"])
def test_workload_full_size(gpu_device, wl):
    say("workload", wl)
    w = make_workload(wl)
    d = upload(w, gpu_device)
    og, lg, _ = run_decode(w, d)
    del d
    torch.cuda.empty_cache()
    o_ref, l_ref = OA.batch_decode(w)
    err = assert_parity(og, lg, o_ref, l_ref, w["o_dtype"], wl)
    print(f"{wl}: max |o - oracle| = {err:.3e}")


@pytest.mark.parametrize("kvd", ["f16", "bf16", "e4m3"])
def test_dtype_decode_legs(gpu_device, kvd):
    say("dtype_decode", kvd)
    w = make_workload("dtype_decode", kvd=kvd)
    d = upload(w, gpu_device)
    og, lg, _ = run_decode(w, d)
    o_ref, l_ref = OA.batch_decode(w)
    assert_parity(og, lg, o_ref, l_ref, "f16", f"dtype-decode workload {kvd}")


def test_dtype_decode_refusals_with_real_tensors(gpu_device):
    """k/v dtype mismatch, integer KV and fp8 output must error, and leave o
    untouched."""
    say("dtype_decode refusals")
    w = make_paged(5, kv_lens=[100, 40], hq=32, hkv=8, d=128, page=16, q="f16", kvd="e4m3")
    d = upload(w, gpu_device)
    o = torch.full((2, 32, 128), 7.0, dtype=torch.float16, device=gpu_device)
    cases = [
        (dict(k_dtype="e4m3", v_dtype="e5m2"), "k has dtype float8_e4m3fn but v has dtype float8_e5m2"),
        (dict(kv_dtype="i8"), "KV cache has dtype int8, which has no float interpretation"),
        (dict(kv_dtype="u8"), "KV cache has dtype uint8"),
    ]
    for kw, frag in cases:
        kv, keep = fi.make_paged_kv(d["k"], d["v"], d["indptr"], d["indices"], d["lpl"], k_scale=w["k_scale"],
                                    v_scale=w["v_scale"], indptr_h=w["indptr"], last_page_len_h=w["last_page_len"], **kw)
        with pytest.raises(fi.FiValueError, match=frag):
            fi.fi_batch_decode_paged(d["q"], kv, o)
    kv, keep = paged_kv(w, d)
    with pytest.raises(fi.FiValueError, match="an fp8 output is not supported"):
        fi.fi_batch_decode_paged(d["q"], kv, o, o_dtype="e4m3")
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)
    # prefill refuses a bf16 cache under an f16 query; decode accepts it (tested above)
    w2 = make_paged(6, qo_lens=[4], prefix_lens=[10], hq=32, hkv=8, d=128, page=16, q="f16", kvd="bf16")
    d2 = upload(w2, gpu_device)
    kv2, keep2 = paged_kv(w2, d2)
    o2 = torch.full((4, 32, 128), 7.0, dtype=torch.float16, device=gpu_device)
    with pytest.raises(fi.FiValueError, match="prefill needs a 2-byte KV cache of the query's dtype"):
        fi.fi_batch_prefill_paged(d2["q"], d2["qo_indptr"], kv2, o2, qo_indptr_h=w2["qo_indptr"])
    torch.cuda.synchronize()
    assert torch.all(o2 == 7.0)


@pytest.mark.parametrize("kvd", ["e4m3fnuz", "e5m2fnuz"])
def test_fnuz_batch_decode_shapes_and_single(gpu_device, kvd):
    """The batch-decode shapes (64 requests of 512..4096 tokens, 32/8 heads,
    page 16 shuffled) over an fnuz cache, every request against the oracle;
    and fi_single_decode over one request's rows."""
    say("fnuz batch_decode shapes", kvd)
    w = make_workload("batch_decode", kvd=kvd)
    d = upload(w, gpu_device)
    og, lg, _ = run_decode(w, d)
    o_ref, l_ref = OA.batch_decode(w)
    assert_parity(og, lg, o_ref, l_ref, "bf16", f"{kvd} batch decode")
    i = 5
    pages = w["indices"][w["indptr"][i]:w["indptr"][i + 1]]
    n = int(w["kv_lens"][i])
    k = torch.from_numpy(np.ascontiguousarray(w["k_pool"][pages].reshape(-1, 8, 128)[:n])).to(gpu_device)
    v = torch.from_numpy(np.ascontiguousarray(w["v_pool"][pages].reshape(-1, 8, 128)[:n])).to(gpu_device)
    q1 = d["q"][i]
    o1 = torch.empty_like(q1)
    l1 = torch.empty(32, dtype=torch.float32, device=gpu_device)
    fi.fi_single_decode(q1, k, v, o1, k_scale=w["k_scale"], v_scale=w["v_scale"], kv_dtype=kvd, lse=l1)
    torch.cuda.synchronize()
    o_s, l_s = OA.single_decode(w["q"][i], "bf16", k.cpu().numpy(), v.cpu().numpy(), kvd, w["k_scale"], w["v_scale"])
    assert_parity(o1.double().cpu().numpy(), l1.double().cpu().numpy(), o_s, l_s, "bf16", f"{kvd} single decode")


def run_decode_fp8q(w: dict, d: dict, *, split=None, workspace=True):
    import os
    B = len(w["kv_lens"])
    o = torch.full((B, w["num_qo_heads"], w["head_dim"]), float("nan"), dtype=T2[w["o_dtype"]], device=gpu_dev(d))
    lse = torch.full((B, w["num_qo_heads"]), float("nan"), dtype=torch.float32, device=gpu_dev(d))
    ws = workspace_for(w, gpu_dev(d)) if workspace else None
    kv, keep = paged_kv(w, d)
    old = os.environ.get("FI_SPLIT_KV")
    try:
        if split is not None:
            os.environ["FI_SPLIT_KV"] = str(split)
        fi.fi_batch_decode_paged_fp8q(d["q"], kv, o, q_dtype=w["q_dtype"], q_scale=w["q_scale"], lse=lse, workspace=ws)
    finally:
        if split is not None:
            if old is None:
                os.environ.pop("FI_SPLIT_KV", None)
            else:
                os.environ["FI_SPLIT_KV"] = old
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def gpu_dev(d):
    return d["q"].device


FP8Q = [
    # (q, kvd, o, page, d, hq, hkv, lens, split)
    ("e4m3", "e4m3", "bf16", 16, 128, 32, 8, (1, 31, 32, 33, 200, 517, 0, 64), None),
    ("e5m2", "e4m3fnuz", "f16", 16, 128, 32, 8, (700, 129, 5), "128"),
    ("e4m3", "e5m2", "f16", 4, 64, 8, 2, (77, 300, 1), None),
    ("e5m2", "e5m2fnuz", "bf16", 64, 128, 64, 8, (1000, 3, 2049), "256"),
]


@pytest.mark.parametrize("case", FP8Q, ids=[f"q{c[0]}-{c[1]}-o{c[2]}-p{c[3]}-d{c[4]}-h{c[5]}x{c[6]}-s{c[8]}" for c in FP8Q])
def test_decode_fp8_query(gpu_device, case):
    """An fp8 query with its q_scale (fi_batch_decode_paged_fp8q) against the
    oracle, and against fi_batch_decode_paged on the same values widened to
    fp16 with q_scale moved into sm_scale."""
    q, kvd, o, page, d_, hq, hkv, lens, split = case
    say("decode fp8 query", case)
    w = make_paged(12, kv_lens=list(lens), hq=hq, hkv=hkv, d=d_, page=page, q=q, kvd=kvd, o=o, extra_pages=2)
    dv = upload(w, gpu_device)
    og, lg = run_decode_fp8q(w, dv, split=split)
    o_ref, l_ref = OA.batch_decode(w)
    assert_parity(og, lg, o_ref, l_ref, o, str(case))
    qw = fp8_table(q)[w["q"]].astype(np.float32)
    w16 = dict(w, q=None, q_dtype="f16", q_scale=1.0)
    d16 = dict(dv, q=torch.from_numpy(qw).to(torch.float16).to(gpu_device))
    o2, l2, _ = run_decode(w16, d16, split=split, sm_scale=OA.default_sm_scale(d_) * w["q_scale"])
    assert np.max(np.abs(og - o2)) <= O_TOL[o] and np.max(np.abs(lg[np.isfinite(lg)] - l2[np.isfinite(l2)])) <= 1e-3


def test_fp8q_prefill_refuses_fnuz(gpu_device):
    """The fp8-query prefill runs the OCP fp8 matrix cores on the raw cache
    codes, so it refuses an fnuz cache with a sentence and leaves o as it was
    (the 2-byte-query prefill reads fnuz caches: test_gpu_prefill)."""
    w = make_paged(8, qo_lens=[4], prefix_lens=[10], hq=8, hkv=2, d=64, page=16, q="e4m3", kvd="e4m3fnuz", o="f16")
    d = upload(w, gpu_device)
    kv, keep = paged_kv(w, d)
    o = torch.full((4, 8, 64), 7.0, dtype=torch.float16, device=gpu_device)
    with pytest.raises(fi.FiValueError, match="an fp8-query prefill runs the OCP fp8 matrix cores"):
        fi.fi_batch_prefill_paged_fp8q(d["q"], d["qo_indptr"], kv, o, q_dtype="e4m3", q_scale=w["q_scale"],
                                       qo_indptr_h=w["qo_indptr"])
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)


# ------------------------------------------------------------------ invariants
def _mid_workload(seed=21, kvd="e4m3", q="bf16", extra_pages=0):
    return make_paged(seed, kv_lens=[1500, 33, 900, 2048, 7, 640], hq=32, hkv=8, d=128, page=16, q=q, kvd=kvd,
                      extra_pages=extra_pages)


def test_determinism_and_page_permutation(gpu_device):
    say("determinism + page permutation")
    w = _mid_workload()
    d = upload(w, gpu_device)
    o1, l1, _ = run_decode(w, d, split="256")
    o2, l2, _ = run_decode(w, d, split="256")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # move every page elsewhere in the pool and remap the indices
    P = w["k_pool"].shape[0]
    perm = np.random.default_rng(3).permutation(P)
    inv = np.argsort(perm)
    w2 = dict(w, k_pool=w["k_pool"][perm], v_pool=w["v_pool"][perm], indices=inv[w["indices"]].astype(np.int32))
    d2 = upload(w2, gpu_device)
    o3, l3, _ = run_decode(w2, d2, split="256")
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


@pytest.mark.parametrize("kvd,q", [("e4m3", "bf16"), ("e5m2", "f16"), ("e4m3fnuz", "f16"), ("e5m2fnuz", "bf16")])
def test_fp8_equals_prewidened_bitwise(gpu_device, kvd, q):
    """fp8 K/V give bit-identical output to the same values stored widened in
    q's 2-byte type, with the same scales."""
    say("prewidened", kvd, q)
    w = _mid_workload(kvd=kvd, q=q)
    d = upload(w, gpu_device)
    o1, l1, _ = run_decode(w, d)
    tab = fp8_table(kvd)
    kw = tab[w["k_pool"]].astype(np.float32)
    vw = tab[w["v_pool"]].astype(np.float32)
    kw[~np.isfinite(kw)] = np.nan
    k2 = torch.from_numpy(kw).to(T2[q]).to(gpu_device)
    v2 = torch.from_numpy(vw).to(T2[q]).to(gpu_device)
    kv, keep = paged_kv(w, d, k=k2, v=v2, kv_dtype=q)
    o2, l2, _ = run_decode(w, d, kv=kv)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("plant", ["none", "some_steps"])
@pytest.mark.parametrize("q", ["f16", "bf16"])
@pytest.mark.parametrize("kvd", ["e4m3fnuz", "e5m2fnuz"])
def test_fnuz_outside_ocp_codes(gpu_device, kvd, q, plant):
    """fnuz decode widens through the OCP converter unless a wave's step holds
    a code with no OCP reading -- e4m3fnuz +-240 (0x7F / 0xFF, OCP NaN),
    e5m2fnuz exponent 0 or 1 with a nonzero magnitude -- and such steps take
    the exact bit form.  With every such code removed (fast form only) and
    with some planted in every third step (both forms in one call), the
    output matches the oracle and is bit-identical to the same values stored
    pre-widened in q's type."""
    say("fnuz outside-OCP codes", kvd, q, plant)
    w = _mid_workload(kvd=kvd, q=q)
    kp, vp = w["k_pool"].copy(), w["v_pool"].copy()
    pages_of = lambda i: w["indices"][w["indptr"][i]:w["indptr"][i + 1]]
    valid = np.zeros(kp.shape[:2], dtype=bool)  # (page, slot) holding a token of some request
    for i, n in enumerate(w["kv_lens"]):
        for t in range(int(n)):
            valid[pages_of(i)[t // 16], t % 16] = True
    vsel = valid[:, :, None, None]
    if kvd == "e4m3fnuz":
        outside = lambda pool: (pool == 0x7F) | (pool == 0xFF)
        repl = lambda pool, sel: pool[sel] - 1  # +-240 -> +-224
        planted = (0x7F, 0xFF)
    else:
        outside = lambda pool: ((pool & 0x78) == 0) & ((pool & 0x7F) != 0)
        repl = lambda pool, sel: 0  # tiny -> +0 (0x80 is the NaN code)
        planted = (0x01, 0x06, 0x85, 0x87)
    for pool in (kp, vp):
        sel = vsel & outside(pool)
        pool[sel] = repl(pool, sel)
    if plant == "some_steps":
        rng = np.random.default_rng(5)
        for i, n in enumerate(w["kv_lens"]):
            for t in range(0, int(n), 48):  # one token in every third 16-token step
                pg, sl = pages_of(i)[t // 16], t % 16
                h, dd = rng.integers(0, 8), rng.integers(0, 128)
                (kp if (t // 48) % 2 == 0 else vp)[pg, sl, h, dd] = planted[rng.integers(0, len(planted))]
    w = dict(w, k_pool=kp, v_pool=vp)
    d = upload(w, gpu_device)
    o1, l1, _ = run_decode(w, d)
    o_ref, l_ref = OA.batch_decode(w)
    assert_parity(o1, l1, o_ref, l_ref, q, f"{kvd} outside-OCP codes {plant}")
    tab = fp8_table(kvd)
    kw = tab[kp].astype(np.float32)
    vw = tab[vp].astype(np.float32)
    kw[~np.isfinite(kw)] = np.nan
    vw[~np.isfinite(vw)] = np.nan
    k2 = torch.from_numpy(kw).to(T2[q]).to(gpu_device)
    v2 = torch.from_numpy(vw).to(T2[q]).to(gpu_device)
    kv, keep = paged_kv(w, d, k=k2, v=v2, kv_dtype=q)
    o2, l2, _ = run_decode(w, d, kv=kv)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_kscale_fold(gpu_device):
    """Scaling k_scale by c equals scaling sm_scale by c; dropping the fold
    would fail the oracle comparison (the A/B check recorded in "fp8 KV cache in
    the in-tree prefill kernel", Test plan)."""
    say("k_scale fold")
    w = _mid_workload(q="f16")
    d = upload(w, gpu_device)
    c = 4.0
    sm = 0.05
    kv_a, ka = paged_kv(w, d, k_scale=w["k_scale"] * c)
    oa, la, _ = run_decode(w, d, kv=kv_a, sm_scale=sm, o_dtype="f16")
    kv_b, kb = paged_kv(w, d)
    ob, lb, _ = run_decode(w, d, kv=kv_b, sm_scale=sm * c, o_dtype="f16")
    assert np.max(np.abs(oa - ob)) <= 2e-3 and np.max(np.abs(la - lb)) <= 1e-4
    w_ref = dict(w, k_scale=w["k_scale"] * c)
    o_ref, l_ref = OA.batch_decode(w_ref, sm_scale=sm)
    assert_parity(oa, la, o_ref, l_ref, "f16", "k_scale fold")
    o_wrong, _ = OA.batch_decode(w, sm_scale=sm)  # the fold left out
    assert np.max(np.abs(oa - o_wrong)) > O_TOL["f16"]


def test_constant_v(gpu_device):
    """Every token carries the same V row: the output is that row times v_scale
    (up to the output rounding)."""
    say("constant V")
    w = _mid_workload(q="f16")
    row = w["v_pool"][w["indices"][0], 0].copy()
    w["v_pool"][:] = row
    d = upload(w, gpu_device)
    o, l, _ = run_decode(w, d, split="256", o_dtype="f16")
    target = fp8_table("e4m3")[row] * w["v_scale"]  # [H_kv, D]
    grp = 32 // 8
    exp = np.repeat(target, grp, axis=0)[None].repeat(o.shape[0], 0)
    np.testing.assert_allclose(o, exp.astype(np.float16).astype(np.float64), rtol=2e-3, atol=1e-6)


@pytest.mark.parametrize("kvd", ["e4m3", "e4m3fnuz", "e5m2fnuz"])
def test_poisoned_pages_stay_finite(gpu_device, kvd):
    """Unused slots and unreferenced pages hold the format's NaN code (0x7F
    OCP, 0x80 fnuz); outputs stay finite, so nothing outside the requests'
    tokens is read."""
    say("poisoned pages", kvd)
    w = _mid_workload(kvd=kvd, extra_pages=50)
    assert np.isnan(fp8_table(kvd)[w["k_pool"][~w["valid"]]]).all()
    d = upload(w, gpu_device)
    o, l, _ = run_decode(w, d, split="128")
    o_ref, l_ref = OA.batch_decode(w)
    assert_parity(o, l, o_ref, l_ref, "bf16", f"poisoned {kvd}")


@pytest.mark.parametrize("split", [None, "128"])
@pytest.mark.parametrize("kvd", ["e4m3", "e4m3fnuz", "e5m2fnuz"])
def test_nan_code_propagates(gpu_device, kvd, split):
    """One K element of one request and kv head set to the format's NaN code
    (0x7F for OCP e4m3, 0x80 for fnuz): the q heads of that kv head in that
    request come out NaN, as in the oracle, and every other output matches it
    -- a NaN in an fnuz cache propagates as one in an OCP cache does."""
    say("NaN code propagates", kvd, split)
    w = _mid_workload(kvd=kvd)
    i, g = 2, 5
    pg = w["indices"][w["indptr"][i] + 3]
    w["k_pool"][pg, 7, g, 17] = NAN_BITS[kvd]
    d = upload(w, gpu_device)
    og, lg, _ = run_decode(w, d, split=split)
    o_ref, l_ref = OA.batch_decode(w)
    bad = np.zeros(og.shape[:2], dtype=bool)
    bad[i, 4 * g:4 * g + 4] = True  # 32 q heads over 8 kv heads
    assert np.isnan(o_ref[bad]).all() and np.isnan(l_ref[bad]).all()
    assert np.isnan(og[bad]).all(), "the rows that read the NaN code are not NaN"
    assert np.isnan(lg[bad]).all()
    assert_parity(og[~bad], lg[~bad], o_ref[~bad], l_ref[~bad], "bf16", f"NaN code {kvd}, other rows")


def test_head_major_pool_layout(gpu_device):
    """A pool stored [num_pages, H_kv, page_size, D] passed through its strides."""
    say("HND layout")
    w = _mid_workload(q="f16")
    d = upload(w, gpu_device)
    k_hnd = d["k"].permute(0, 2, 1, 3).contiguous()  # [P, H, page, D]
    v_hnd = d["v"].permute(0, 2, 1, 3).contiguous()
    kv, keep = paged_kv(w, d, k=k_hnd.permute(0, 2, 1, 3), v=v_hnd.permute(0, 2, 1, 3))
    o, l, _ = run_decode(w, d, kv=kv)
    o_ref, l_ref = OA.batch_decode(w)
    assert_parity(o, l, o_ref, l_ref, "f16", "HND")


def test_split_and_unsplit_agree(gpu_device):
    say("split vs unsplit")
    w = _mid_workload()
    d = upload(w, gpu_device)
    o_ref, l_ref = OA.batch_decode(w)
    for split in ("off", "128", "384", "auto"):
        o, l, _ = run_decode(w, d, split=split)
        assert_parity(o, l, o_ref, l_ref, "bf16", f"split={split}")
    o, l, _ = run_decode(w, d, workspace=False)
    assert_parity(o, l, o_ref, l_ref, "bf16", "no workspace")


@pytest.mark.parametrize("batch", [900, 1100])
def test_decode_large_batch(gpu_device, batch):
    """Batches past the limits of the planner's fast paths: above 768
    requests the token prefix sums no longer travel in the kernel arguments
    and every workgroup scans the page table itself; above 1024 the planner
    falls back to fixed chunks.  Short, ragged requests (some empty) against
    the oracle."""
    say("decode large batch", batch)
    rng = np.random.default_rng(batch)
    lens = rng.integers(0, 300, size=batch)
    lens[::97] = 0
    w = make_paged(batch, kv_lens=list(lens), hq=8, hkv=2, d=64, page=16, q="bf16", kvd="e4m3")
    d = upload(w, gpu_device)
    og, lg, _ = run_decode(w, d)
    o_ref, l_ref = OA.batch_decode(w)
    assert_parity(og, lg, o_ref, l_ref, "bf16", f"decode batch {batch}")


def test_decode_page1_many_windows(gpu_device):
    """page_size 1 with 2500 pages in one request: the page ids are staged in
    three LDS windows of 1024 pages."""
    say("decode page 1, 2500 pages")
    w = make_paged(41, kv_lens=[2500, 7, 1100], hq=16, hkv=4, d=128, page=1, q="f16", kvd="e5m2")
    d = upload(w, gpu_device)
    for split in (None, "128"):
        og, lg, _ = run_decode(w, d, split=split)
        o_ref, l_ref = OA.batch_decode(w)
        assert_parity(og, lg, o_ref, l_ref, "f16", f"decode page 1, split {split}")
