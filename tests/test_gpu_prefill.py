"""GPU parity tests for batched paged prefill (causal and not), through the C
ABI, against the float64 oracle.

Cases: the causal-prefill workload (16 requests, qo 256..1024, prefix 0..2048, 32/8 heads, d 128) at full size, every
request compared element by element; a matrix of
small shapes (GQA groups 1, 2, 3, 4, 8, 32; head_dim 64 and 128; page sizes 1 to
128; fp8 and same-type 2-byte KV; causal and non-causal; ragged query and
prefix lengths that leave partial tiles); rows with no visible key; requests
without queries or without keys; decode equal to prefill with one query per
request; run-to-run determinism and page-permutation invariance (bitwise);
fp8 (OCP and fnuz) equal to the same values stored in the 2-byte type
(bitwise); fnuz caches in the shape matrix; constant V;
a head-major pool through its strides; 200 requests, more than the geometry
the kernel arguments hold; 800 requests, more (request, query block) pairs
than the dispatch order in the kernel arguments holds; NaN codes in K and V.
"""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from oracle.fp8 import fp8_table
from workloads import NAN_BITS, make_paged, make_workload
from attention_paged_fp8_amd import fi
from gpu_util import T2, assert_parity, assert_parity_nan, paged_kv, plant_codes, run_decode, run_prefill, say, upload

pytestmark = pytest.mark.gpu

SMALL = [
    # (kvd, q, o, page, d, hq, hkv, qo, prefix, causal)
    ("e4m3", "f16", "f16", 16, 128, 32, 8, (1, 37, 130, 64), (0, 100, 5, 300), True),
    ("e4m3", "f16", "f16", 16, 128, 32, 8, (1, 37, 130, 64), (0, 100, 5, 300), False),
    ("e5m2", "bf16", "bf16", 64, 128, 16, 8, (200, 33), (70, 0), True),       # group 2
    ("e4m3", "bf16", "f16", 4, 64, 8, 8, (129, 3, 257), (1, 64, 0), True),    # group 1
    ("e4m3", "f16", "bf16", 1, 64, 12, 4, (45, 90), (10, 0), True),           # group 3
    ("e5m2", "f16", "f16", 32, 128, 64, 8, (100, 65), (40, 1), True),         # group 8 (two head subgroups)
    ("f16", "f16", "f16", 16, 128, 32, 8, (77, 256), (3, 128), True),
    ("bf16", "bf16", "bf16", 8, 64, 4, 2, (150,), (200,), True),
    ("e4m3", "bf16", "bf16", 128, 128, 32, 8, (70, 300), (400, 2), False),  # page 128, non-causal with prefix
    ("e5m2", "f16", "f16", 128, 64, 16, 4, (129, 64), (0, 190), True),
    ("e4m3", "f16", "f16", 16, 128, 32, 1, (65, 3), (100, 0), True),       # group 32: 8 head subgroups
    ("e5m2", "bf16", "bf16", 1, 64, 2, 2, (300,), (0,), True),             # page 1, one q head per kv head
    ("e4m3", "f16", "f16", 16, 128, 8, 8, (700,), (1300,), False),         # long non-causal with a prefix
    # fnuz caches (the gfx942 layouts; widened exactly from the bits)
    ("e4m3fnuz", "f16", "f16", 16, 128, 32, 8, (1, 37, 130, 64), (0, 100, 5, 300), True),
    ("e4m3fnuz", "bf16", "bf16", 4, 64, 8, 2, (129, 3), (1, 64), False),
    ("e5m2fnuz", "bf16", "f16", 64, 128, 16, 8, (200, 33), (70, 0), True),
    ("e5m2fnuz", "f16", "bf16", 1, 64, 12, 4, (45, 90), (10, 0), True),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-q{c[1]}-o{c[2]}-p{c[3]}-d{c[4]}-h{c[5]}x{c[6]}-c{int(c[9])}" for c in SMALL])
def test_prefill_small(gpu_device, case):
    kvd, q, o, page, d, hq, hkv, qo, prefix, causal = case
    say("prefill small", case)
    w = make_paged(31, qo_lens=list(qo), prefix_lens=list(prefix), hq=hq, hkv=hkv, d=d, page=page, q=q, kvd=kvd,
                   o=o, extra_pages=2)
    dv = upload(w, gpu_device)
    og, lg, _ = run_prefill(w, dv, causal=causal)
    o_ref, l_ref = OA.batch_prefill(w, causal=causal)
    assert_parity(og, lg, o_ref, l_ref, o, str(case))


def test_causal_prefill_full_size(gpu_device):
    """The causal-prefill workload at full size: all 16 requests, every
    element of o and lse against the float64 oracle."""
    say("causal_prefill")
    w = make_workload("causal_prefill")
    d = upload(w, gpu_device)
    og, lg, _ = run_prefill(w, d, causal=True)
    og2, lg2, _ = run_prefill(w, d, causal=True)
    assert np.array_equal(og, og2) and np.array_equal(lg, lg2), "prefill is not deterministic"
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    err = assert_parity(og, lg, o_ref, l_ref, "f16", "causal-prefill workload")
    print(f"causal-prefill workload: max |o - oracle| = {err:.3e}")


@pytest.mark.parametrize("kvd,q", [("e4m3", "f16"), ("e5m2", "bf16"), ("e4m3fnuz", "f16"), ("e5m2fnuz", "bf16")])
def test_prefill_nan_code_propagates(gpu_device, kvd, q):
    """The format's NaN code in one K element of a key that only the later
    query rows see (causal mask), and in one V element of a prefix key that
    every row sees: the oracle's NaN outputs -- whole rows of that kv head's
    q heads from the first row that sees the key, and the V element's column
    of every row -- are NaN, and every other output matches it."""
    say("prefill NaN code", kvd, q)
    w = make_paged(37, qo_lens=[40, 130, 64], prefix_lens=[10, 300, 0], hq=32, hkv=8, d=128, page=16, q=q,
                   kvd=kvd, o=q, extra_pages=2)
    plant_codes(w, 1, [("k_pool", 350, 5, 17, NAN_BITS[kvd]), ("v_pool", 100, 2, 40, NAN_BITS[kvd])])
    dv = upload(w, gpu_device)
    og, lg, _ = run_prefill(w, dv, causal=True)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    assert np.isnan(l_ref).sum() == (130 - 50) * 4  # rows 50.. of request 1 see key 350
    assert_parity_nan(og, lg, o_ref, l_ref, q, f"NaN code {kvd}")


def test_rows_without_visible_keys(gpu_device):
    """qo_len > kv_len under a causal mask aligned to the kv end: the first
    qo_len - kv_len rows see nothing (o = 0, lse = -inf)."""
    say("prefill empty rows")
    w = make_paged(41, qo_lens=[20, 5], kv_lens=[12, 5], hq=8, hkv=2, d=128, page=16, q="f16", kvd="e4m3")
    d = upload(w, gpu_device)
    og, lg, _ = run_prefill(w, d, causal=True)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    assert np.all(og[:8] == 0) and np.all(np.isneginf(lg[:8]))
    assert_parity(og, lg, o_ref, l_ref, "f16", "empty rows")


def test_decode_equals_prefill_one_query(gpu_device):
    say("decode vs prefill qo_len=1")
    w = make_paged(43, kv_lens=[1, 100, 700, 2000], hq=32, hkv=8, d=128, page=16, q="bf16", kvd="e4m3")
    d = upload(w, gpu_device)
    od, ld, _ = run_decode(w, d)
    op, lp, _ = run_prefill(w, d, causal=True)
    assert np.max(np.abs(od - op)) <= 2e-2 and np.max(np.abs(ld - lp)) <= 1e-3
    o_ref, l_ref = OA.batch_decode(w)
    assert_parity(op, lp, o_ref, l_ref, "bf16", "prefill at qo_len=1")


# ------------------------------------------------------------------ invariants
def _prefill_mid(seed=51, kvd="e4m3", q="f16", extra_pages=0):
    return make_paged(seed, qo_lens=[300, 17, 64, 129], prefix_lens=[700, 0, 1000, 63], hq=32, hkv=8, d=128,
                      page=16, q=q, kvd=kvd, extra_pages=extra_pages)


def test_prefill_page_permutation_bitwise(gpu_device):
    """Moving every page elsewhere in the pool (indices remapped) changes no bit."""
    say("prefill page permutation")
    w = _prefill_mid(extra_pages=20)
    d = upload(w, gpu_device)
    o1, l1, _ = run_prefill(w, d, causal=True)
    P = w["k_pool"].shape[0]
    perm = np.random.default_rng(5).permutation(P)
    inv = np.argsort(perm)
    w2 = dict(w, k_pool=w["k_pool"][perm], v_pool=w["v_pool"][perm], indices=inv[w["indices"]].astype(np.int32))
    o2, l2, _ = run_prefill(w2, upload(w2, gpu_device), causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    assert_parity(o1, l1, o_ref, l_ref, "f16", "prefill page permutation")


@pytest.mark.parametrize("kvd,q", [("e4m3", "f16"), ("e5m2", "bf16"), ("e4m3fnuz", "bf16"), ("e5m2fnuz", "f16")])
def test_prefill_fp8_equals_prewidened_bitwise(gpu_device, kvd, q):
    """fp8 K/V give bit-identical output to the same values stored widened in
    q's 2-byte type (the tiles the kernel builds are the same)."""
    say("prefill prewidened", kvd, q)
    w = _prefill_mid(kvd=kvd, q=q)
    d = upload(w, gpu_device)
    o1, l1, _ = run_prefill(w, d, causal=True)
    tab = fp8_table(kvd)
    kw = tab[w["k_pool"]].astype(np.float32)
    vw = tab[w["v_pool"]].astype(np.float32)
    k2 = torch.from_numpy(kw).to(T2[q]).to(gpu_device)
    v2 = torch.from_numpy(vw).to(T2[q]).to(gpu_device)
    kv, keep = paged_kv(w, d, k=k2, v=v2, kv_dtype=q)
    o2, l2, _ = run_prefill(w, d, causal=True, kv=kv)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("plant", ["none", "some_tiles"])
@pytest.mark.parametrize("kvd,q", [("e4m3fnuz", "bf16"), ("e4m3fnuz", "f16"), ("e5m2fnuz", "bf16"), ("e5m2fnuz", "f16")])
def test_prefill_fnuz_outside_ocp_codes(gpu_device, kvd, q, plant):
    """fnuz prefill widens a wave's K or V tile through the OCP converter
    unless the tile holds a code with no OCP reading (e4m3fnuz +-240,
    e5m2fnuz exponent 0 or 1 with a nonzero magnitude); such tiles take the
    exact bit form.  With every such code removed (fast form only) and with
    some planted every 160 tokens (both forms in one call), the output matches
    the oracle and is bit-identical to the same values stored pre-widened."""
    say("prefill fnuz outside-OCP codes", kvd, q, plant)
    w = _prefill_mid(kvd=kvd, q=q)
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
    if plant == "some_tiles":
        rng = np.random.default_rng(6)
        for i, n in enumerate(w["kv_lens"]):
            for t in range(5, int(n), 160):
                pg, sl = pages_of(i)[t // 16], t % 16
                h, dd = rng.integers(0, 8), rng.integers(0, 128)
                (kp if (t // 160) % 2 == 0 else vp)[pg, sl, h, dd] = planted[rng.integers(0, len(planted))]
    w = dict(w, k_pool=kp, v_pool=vp)
    d = upload(w, gpu_device)
    o1, l1, _ = run_prefill(w, d, causal=True)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    assert_parity(o1, l1, o_ref, l_ref, w["o_dtype"], f"prefill {kvd} outside-OCP codes {plant}")
    tab = fp8_table(kvd)
    k2 = torch.from_numpy(tab[kp].astype(np.float32)).to(T2[q]).to(gpu_device)
    v2 = torch.from_numpy(tab[vp].astype(np.float32)).to(T2[q]).to(gpu_device)
    kv, keep = paged_kv(w, d, k=k2, v=v2, kv_dtype=q)
    o2, l2, _ = run_prefill(w, d, causal=True, kv=kv)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_prefill_constant_v(gpu_device):
    """Every token carries the same V row: each output row is that row times
    v_scale (up to the output rounding), causal mask or not."""
    say("prefill constant V")
    w = _prefill_mid()
    row = w["v_pool"][w["indices"][0], 0].copy()
    w["v_pool"][:] = row
    d = upload(w, gpu_device)
    target = fp8_table("e4m3")[row] * w["v_scale"]  # [H_kv, D]
    exp = np.repeat(target, 32 // 8, axis=0)
    for causal in (True, False):
        o, l, _ = run_prefill(w, d, causal=causal)
        np.testing.assert_allclose(o, np.broadcast_to(exp.astype(np.float16).astype(np.float64), o.shape),
                                   rtol=2e-3, atol=1e-6)


def test_prefill_head_major_pool_layout(gpu_device):
    """A pool stored [num_pages, H_kv, page_size, D] passed through its strides."""
    say("prefill HND layout")
    w = _prefill_mid(q="bf16")
    d = upload(w, gpu_device)
    k_hnd = d["k"].permute(0, 2, 1, 3).contiguous()
    v_hnd = d["v"].permute(0, 2, 1, 3).contiguous()
    kv, keep = paged_kv(w, d, k=k_hnd.permute(0, 2, 1, 3), v=v_hnd.permute(0, 2, 1, 3))
    o, l, _ = run_prefill(w, d, causal=True, kv=kv)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    assert_parity(o, l, o_ref, l_ref, "bf16", "prefill HND")


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_requests_without_queries_or_keys(gpu_device, causal):
    """Requests with qo_len 0 produce nothing; requests with kv_len 0 give o = 0
    and lse = -inf for every row; the others are unaffected."""
    say("prefill empty requests", causal)
    w = make_paged(61, qo_lens=[0, 40, 13, 0, 7], kv_lens=[5, 0, 200, 0, 7], hq=8, hkv=2, d=64, page=16,
                   q="bf16", kvd="e5m2")
    d = upload(w, gpu_device)
    o, l, _ = run_prefill(w, d, causal=causal)
    assert np.all(o[0:40] == 0) and np.all(np.isneginf(l[0:40]))
    o_ref, l_ref = OA.batch_prefill(w, causal=causal)
    assert_parity(o, l, o_ref, l_ref, "bf16", "prefill empty requests")


def test_prefill_geometry_from_device(gpu_device):
    """200 short requests: their (request, query block) pairs fit the dispatch
    order in the kernel arguments (512) but their geometry does not (96), so
    the workgroups read each request's rows and pages from the device arrays;
    against the oracle."""
    say("prefill 200 requests")
    rng = np.random.default_rng(200)
    qo = rng.integers(1, 65, size=200)
    prefix = rng.integers(0, 200, size=200)
    w = make_paged(200, qo_lens=list(qo), prefix_lens=list(prefix), hq=8, hkv=2, d=128, page=16, q="f16", kvd="e4m3",
                   o="f16", extra_pages=2)
    dv = upload(w, gpu_device)
    og, lg, _ = run_prefill(w, dv, causal=True)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    assert_parity(og, lg, o_ref, l_ref, "f16", "200 short requests")


def test_prefill_many_query_blocks(gpu_device):
    """More (request, query block) pairs than the dispatch order carried in the
    kernel arguments holds (512): the kernel then walks the grid in request
    order.  800 short requests, one query block each, against the oracle."""
    say("prefill 800 requests")
    rng = np.random.default_rng(800)
    qo = rng.integers(1, 65, size=800)
    prefix = rng.integers(0, 100, size=800)
    w = make_paged(800, qo_lens=list(qo), prefix_lens=list(prefix), hq=8, hkv=8, d=64, page=16, q="f16", kvd="e4m3")
    d = upload(w, gpu_device)
    og, lg, _ = run_prefill(w, d, causal=True)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    assert_parity(og, lg, o_ref, l_ref, "f16", "prefill 800 requests")


# ------------------------------------------------------------------ byte offsets past 4 GiB
def _token_major_pool(w: dict, device, stride_token_bytes: int):
    """The workload's pages placed in token-major pools ([page_size, pages,
    H_kv, D] in memory, so stride_token = pages * H_kv * D elements) with so
    many pages that one token stride is stride_token_bytes; the used pages go
    to the top of the pool.  Returns (k, v as [pages, page_size, H_kv, D]
    strided views, remapped indices)."""
    page, hkv, d = w["page_size"], w["num_kv_heads"], w["head_dim"]
    row = hkv * d  # fp8: bytes of one (page, slot)
    n_big = -(-stride_token_bytes // row)
    ids = (n_big - 1 - 3 * np.arange(w["k_pool"].shape[0])).astype(np.int64)  # spread near the top
    assert ids.min() >= 0
    out = []
    for name in ("k_pool", "v_pool"):
        big = torch.zeros((page, n_big, hkv, d), dtype=torch.uint8, device=device)
        small = torch.from_numpy(np.ascontiguousarray(w[name])).to(device)  # [P, page, H, D]
        big[:, torch.from_numpy(ids).to(device)] = small.permute(1, 0, 2, 3)
        out.append(big.permute(1, 0, 2, 3))  # [n_big, page, H, D] view
    return out[0], out[1], ids[w["indices"]].astype(np.int32)


def test_slot_offsets_past_4gib(gpu_device):
    """A token-major pool at page 128 whose token stride is 35 MB: slot 127 of a
    page lies 4.4 GB past the page's first slot, so the in-page byte offset
    (slot x token stride) passes 4 GiB.  Prefill (2-byte and fp8 query) and
    decode read the right rows: parity with the oracle on the compact pool."""
    say("slot offsets past 4 GiB")
    stride = 35 << 20
    assert 127 * stride > (1 << 32)
    w = make_paged(57, qo_lens=[40, 130], prefix_lens=[300, 120], hq=8, hkv=2, d=128, page=128, q="f16", kvd="e4m3")
    d = upload(w, gpu_device)
    k, v, idx = _token_major_pool(w, gpu_device, stride)
    assert k.stride(1) * 127 > (1 << 32)
    ind = torch.from_numpy(idx).to(gpu_device)
    kv, keep = fi.make_paged_kv(k, v, d["indptr"], ind, d["lpl"], k_scale=w["k_scale"], v_scale=w["v_scale"],
                                kv_dtype="e4m3", indptr_h=w["indptr"], last_page_len_h=w["last_page_len"])
    og, lg, _ = run_prefill(w, d, causal=True, kv=kv)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    assert_parity(og, lg, o_ref, l_ref, "f16", "prefill, token-major pool")
    # the fp8-query prefill on the same pool
    w8 = make_paged(57, qo_lens=[40, 130], prefix_lens=[300, 120], hq=8, hkv=2, d=128, page=128, q="e4m3",
                    kvd="e4m3")
    q8 = torch.from_numpy(np.ascontiguousarray(w8["q"])).to(gpu_device)
    o8 = torch.full(og.shape, float("nan"), dtype=torch.float16, device=gpu_device)
    l8 = torch.full(lg.shape, float("nan"), dtype=torch.float32, device=gpu_device)
    kv8, keep8 = fi.make_paged_kv(k, v, d["indptr"], ind, d["lpl"], k_scale=w8["k_scale"], v_scale=w8["v_scale"],
                                  kv_dtype="e4m3", indptr_h=w["indptr"], last_page_len_h=w["last_page_len"])
    fi.fi_batch_prefill_paged_fp8q(q8, d["qo_indptr"], kv8, o8, q_dtype="e4m3", q_scale=w8["q_scale"], o_dtype="f16",
                                   causal=True, lse=l8, qo_indptr_h=w["qo_indptr"])
    torch.cuda.synchronize()
    o_ref8, l_ref8 = OA.batch_prefill(w8, causal=True)
    assert_parity(o8.double().cpu().numpy(), l8.double().cpu().numpy(), o_ref8, l_ref8, "f16",
                  "fp8-query prefill, token-major pool")
    # decode, one query per request, over the same pages
    wd = dict(w, qo_indptr=np.arange(3, dtype=np.int32), qo_lens=np.ones(2, dtype=np.int64),
              q=w["q"][w["qo_indptr"][1:] - 1])
    dd = dict(d, q=dev_q(wd, gpu_device))
    od, ld, _ = run_decode(wd, dd, kv=kv)
    o_refd, l_refd = OA.batch_decode(wd)
    assert_parity(od, ld, o_refd, l_refd, "f16", "decode, token-major pool")
    del k, v, kv, keep, kv8, keep8
    torch.cuda.empty_cache()


def dev_q(w, device):
    return torch.from_numpy(np.ascontiguousarray(w["q"]).view(np.int16)).view(T2[w["q_dtype"]]).to(device)
