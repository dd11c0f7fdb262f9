"""GPU tests of fi_batch_pod_paged: a prefill batch and a decode batch in one
launch, through the C ABI, against the float64 oracle.

Cases: a matrix of mixed batches (f16 and bf16 queries and outputs, OCP and
fnuz fp8 and same-type 2-byte caches, head_dim 64 and 128, GQA groups 1 to
8, page sizes 1 to 128, causal and not, with and without a split-KV
workspace, empty requests in both phases); the prefill phase bit-identical
to fi_batch_prefill_paged on the same inputs; one phase empty; the two
phases over the same pools with different page tables; and at full size the
causal-prefill workload with the batch-decode shapes in f16 (16 prefill and
64 decode requests) in one call, every element against the oracle; NaN codes
in both phases; phases larger than the geometry (48 requests) and prefix sums
(256 requests) one launch's arguments carry.
"""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from attention_paged_fp8_amd import fi
from workloads import NAN_BITS, make_paged, make_workload
from gpu_util import T2, assert_parity, assert_parity_nan, paged_kv, plant_codes, say, upload, workspace_for

pytestmark = pytest.mark.gpu


def run_pod(wp, dp, wd, dd, *, causal=True, workspace=True, kv_p=None, kv_d=None):
    """Both phases in one call; returns ((o_p, lse_p), (o_d, lse_d)) as float64."""
    dev = dp["q"].device if wp is not None else dd["q"].device
    od = (wp or wd)["o_dtype"]
    H, D = (wp or wd)["num_qo_heads"], (wp or wd)["head_dim"]
    Tp = int(wp["qo_indptr"][-1]) if wp is not None else 0
    Bd = len(wd["kv_lens"]) if wd is not None else 0
    o_p = torch.full((Tp, H, D), float("nan"), dtype=T2[od], device=dev)
    l_p = torch.full((Tp, H), float("nan"), dtype=torch.float32, device=dev)
    o_d = torch.full((Bd, H, D), float("nan"), dtype=T2[od], device=dev)
    l_d = torch.full((Bd, H), float("nan"), dtype=torch.float32, device=dev)
    keep = []
    if kv_p is None:
        kv_p, k1 = paged_kv(wp, dp) if wp is not None else paged_kv(wd, dd)
        keep.append(k1)
    if kv_d is None:
        kv_d, k2 = paged_kv(wd, dd) if wd is not None else paged_kv(wp, dp)
        keep.append(k2)
    ws = workspace_for(wd, dev) if (workspace and wd is not None) else None
    q_p = dp["q"] if wp is not None else None
    qo = dp["qo_indptr"] if wp is not None else torch.zeros(1, dtype=torch.int32, device=dev)
    qo_h = wp["qo_indptr"] if wp is not None else np.zeros(1, np.int32)
    q_d = dd["q"] if wd is not None else torch.empty((0, H, D), dtype=T2[(wp or wd)["q_dtype"]], device=dev)
    fi.fi_batch_pod_paged(q_p, qo, kv_p, o_p, q_d, kv_d, o_d, causal=causal, lse_p=l_p, lse_d=l_d,
                          q_dtype=(wp or wd)["q_dtype"], o_dtype=od, qo_indptr_h=qo_h, batch_d=Bd, num_qo_heads=H,
                          workspace=ws)
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    return (f(o_p), f(l_p)), (f(o_d), f(l_d))


CASES = [
    # (kvd, q, o, page, d, hq, hkv, prefill qo, prefill prefix, decode kv lens, causal, workspace)
    ("e4m3", "f16", "f16", 16, 128, 32, 8, (1, 37, 130, 64), (0, 100, 5, 300), (1, 700, 33, 2048, 0, 513), True, True),
    ("e4m3", "bf16", "bf16", 16, 128, 32, 8, (300, 17), (700, 0), (1500, 2, 900), True, False),
    ("e5m2", "bf16", "f16", 64, 128, 16, 8, (200, 33), (70, 0), (1000, 3, 2049), False, True),
    ("e4m3", "f16", "bf16", 4, 64, 8, 8, (129, 3, 257), (1, 64, 0), (77, 300, 1), True, True),
    ("e5m2", "f16", "f16", 1, 64, 12, 4, (45, 90), (10, 0), (9, 40, 130), True, True),
    ("f16", "f16", "f16", 16, 128, 32, 8, (77, 256), (3, 128), (400, 65, 1), True, True),
    ("bf16", "bf16", "bf16", 8, 64, 4, 2, (150,), (200,), (257, 31), True, True),
    ("e4m3", "f16", "f16", 128, 128, 64, 8, (100, 65), (40, 1), (1000, 3, 2049), True, True),  # group 8
    ("e4m3fnuz", "f16", "f16", 16, 128, 32, 8, (1, 37, 130), (0, 100, 5), (1, 31, 517, 0, 64), True, True),
    ("e5m2fnuz", "bf16", "bf16", 32, 128, 16, 16, (65, 3), (100, 0), (55, 1, 1024), True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-q{c[1]}-o{c[2]}-p{c[3]}-d{c[4]}-h{c[5]}x{c[6]}-c{int(c[10])}-ws{int(c[11])}"
                                             for c in CASES])
def test_pod_small(gpu_device, case):
    kvd, q, o, page, d, hq, hkv, qo, prefix, dec, causal, ws = case
    say("pod small", case)
    wp = make_paged(71, qo_lens=list(qo), prefix_lens=list(prefix), hq=hq, hkv=hkv, d=d, page=page, q=q, kvd=kvd, o=o,
                    extra_pages=2)
    wd = make_paged(72, kv_lens=list(dec), hq=hq, hkv=hkv, d=d, page=page, q=q, kvd=kvd, o=o, extra_pages=3)
    dp, dd = upload(wp, gpu_device), upload(wd, gpu_device)
    (op, lp), (od, ld) = run_pod(wp, dp, wd, dd, causal=causal, workspace=ws)
    o_ref, l_ref = OA.batch_prefill(wp, causal=causal)
    assert_parity(op, lp, o_ref, l_ref, o, f"pod prefill phase {case}")
    o_ref, l_ref = OA.batch_decode(wd)
    assert_parity(od, ld, o_ref, l_ref, o, f"pod decode phase {case}")
    for i, n in enumerate(dec):
        if n == 0:
            assert np.all(od[i] == 0) and np.all(np.isneginf(ld[i]))
    # the prefill phase is the prefill call's work, item for item: identical bits
    kv, keep = paged_kv(wp, dp)
    o2 = torch.full(op.shape, float("nan"), dtype=T2[o], device=gpu_device)
    l2 = torch.full(lp.shape, float("nan"), dtype=torch.float32, device=gpu_device)
    fi.fi_batch_prefill_paged(dp["q"], dp["qo_indptr"], kv, o2, causal=causal, lse=l2, qo_indptr_h=wp["qo_indptr"])
    torch.cuda.synchronize()
    assert np.array_equal(op, o2.double().cpu().numpy()) and np.array_equal(lp, l2.double().cpu().numpy())


@pytest.mark.parametrize("order,wg", [("prefill_first", None), ("decode_first", "512"), ("decode_first", "16")])
def test_pod_dispatch_orders(gpu_device, monkeypatch, order, wg):
    """Both dispatch orders and decode shares far from the default give the
    same results (the prefill phase bit for bit)."""
    say("pod order", order, wg)
    monkeypatch.setenv("FI_POD_ORDER", order)
    if wg:
        monkeypatch.setenv("FI_POD_DECODE_WG", wg)
    wp = make_paged(77, qo_lens=[300, 17, 129], prefix_lens=[700, 0, 63], hq=32, hkv=8, d=128, page=16, q="f16",
                    kvd="e4m3")
    wd = make_paged(78, kv_lens=[1500, 33, 900, 0, 640], hq=32, hkv=8, d=128, page=16, q="f16", kvd="e4m3")
    dp, dd = upload(wp, gpu_device), upload(wd, gpu_device)
    (op, lp), (od, ld) = run_pod(wp, dp, wd, dd)
    o_ref, l_ref = OA.batch_prefill(wp, causal=True)
    assert_parity(op, lp, o_ref, l_ref, "f16", f"pod {order} {wg}, prefill")
    o_ref, l_ref = OA.batch_decode(wd)
    assert_parity(od, ld, o_ref, l_ref, "f16", f"pod {order} {wg}, decode")


def test_pod_one_phase_empty(gpu_device):
    say("pod one phase empty")
    wp = make_paged(73, qo_lens=[90, 20], prefix_lens=[30, 0], hq=8, hkv=2, d=128, page=16, q="f16", kvd="e4m3")
    wd = make_paged(74, kv_lens=[300, 5, 1200], hq=8, hkv=2, d=128, page=16, q="f16", kvd="e4m3")
    dp, dd = upload(wp, gpu_device), upload(wd, gpu_device)
    (op, lp), _ = run_pod(wp, dp, None, None)
    o_ref, l_ref = OA.batch_prefill(wp, causal=True)
    assert_parity(op, lp, o_ref, l_ref, "f16", "pod, prefill only")
    _, (od, ld) = run_pod(None, None, wd, dd)
    o_ref, l_ref = OA.batch_decode(wd)
    assert_parity(od, ld, o_ref, l_ref, "f16", "pod, decode only")


def test_pod_phases_share_pools(gpu_device):
    """kv_p and kv_d over the same K/V pools with their own page tables: the
    decode requests read pages of the prefill requests (a served batch where
    some requests decode while others prefill)."""
    say("pod shared pools")
    wp = make_paged(75, qo_lens=[100, 260, 7], prefix_lens=[500, 0, 60], hq=32, hkv=8, d=128, page=16, q="bf16",
                    kvd="e4m3", extra_pages=4)
    dp = upload(wp, gpu_device)
    # decode requests: request 1's pages, request 0's first 20 pages, request 2's pages
    ip, ix, lp_ = wp["indptr"], wp["indices"], wp["last_page_len"]
    pages = [ix[ip[1]:ip[2]], ix[ip[0]:ip[0] + 20], ix[ip[2]:ip[3]]]
    lens = [int(wp["kv_lens"][1]), 20 * 16, int(wp["kv_lens"][2])]
    wd = dict(wp)
    wd["indptr"] = np.concatenate([[0], np.cumsum([len(x) for x in pages])]).astype(np.int32)
    wd["indices"] = np.concatenate(pages).astype(np.int32)
    wd["last_page_len"] = np.array([lp_[1], 16, lp_[2]], np.int32)
    wd["kv_lens"] = np.array(lens, np.int64)
    wd["qo_indptr"] = np.arange(4, dtype=np.int32)
    wd["qo_lens"] = np.ones(3, np.int64)
    wd["q"] = make_paged(76, kv_lens=[1, 1, 1], hq=32, hkv=8, d=128, page=16, q="bf16", kvd="e4m3")["q"]
    dd = upload(wd, gpu_device)
    kv_d, keep = paged_kv(wd, dd, k=dp["k"], v=dp["v"])  # the prefill phase's pools, the decode phase's table
    (op, lp), (od, ld) = run_pod(wp, dp, wd, dd, kv_d=kv_d)
    o_ref, l_ref = OA.batch_prefill(wp, causal=True)
    assert_parity(op, lp, o_ref, l_ref, "bf16", "pod shared pools, prefill")
    o_ref, l_ref = OA.batch_decode(wd)
    assert_parity(od, ld, o_ref, l_ref, "bf16", "pod shared pools, decode")


def test_pod_full_size(gpu_device):
    """The causal-prefill workload (16 requests) and the batch-decode shapes
    with an f16 query over e4m3 (64 requests; the dtype-decode workload's e4m3
    leg) in one call: every element of both phases against the oracle."""
    say("pod full size")
    wp = make_workload("causal_prefill")
    wd = make_workload("dtype_decode", kvd="e4m3")
    dp, dd = upload(wp, gpu_device), upload(wd, gpu_device)
    (op, lp), (od, ld) = run_pod(wp, dp, wd, dd)
    del dp, dd
    torch.cuda.empty_cache()
    o_ref, l_ref = OA.batch_prefill(wp, causal=True)
    e1 = assert_parity(op, lp, o_ref, l_ref, "f16", "pod full size, prefill phase")
    o_ref, l_ref = OA.batch_decode(wd)
    e2 = assert_parity(od, ld, o_ref, l_ref, "f16", "pod full size, decode phase")
    print(f"pod full size: max |o - oracle| prefill {e1:.3e}, decode {e2:.3e}")


@pytest.mark.parametrize("ws", [True, False])
@pytest.mark.parametrize("kvd", ["e4m3", "e4m3fnuz"])
def test_pod_nan_code_propagates(gpu_device, kvd, ws):
    """The format's NaN code planted in both phases: in the prefill batch a K
    element of a key only the later rows see and a V element of a prefix key,
    in the decode batch a K element of one request (split across pieces or
    not).  Exactly the oracle's NaN outputs are NaN in both phases, and every
    other output matches it."""
    say("pod NaN code", kvd, ws)
    wp = make_paged(73, qo_lens=[40, 130, 64], prefix_lens=[10, 300, 0], hq=32, hkv=8, d=128, page=16, q="f16",
                    kvd=kvd, o="f16", extra_pages=2)
    wd = make_paged(74, kv_lens=[700, 2048, 33, 1500], hq=32, hkv=8, d=128, page=16, q="f16", kvd=kvd, o="f16",
                    extra_pages=3)
    plant_codes(wp, 1, [("k_pool", 350, 5, 17, NAN_BITS[kvd]), ("v_pool", 100, 2, 40, NAN_BITS[kvd])])
    plant_codes(wd, 1, [("k_pool", 1200, 3, 9, NAN_BITS[kvd])])
    dp, dd = upload(wp, gpu_device), upload(wd, gpu_device)
    (op, lp), (od, ld) = run_pod(wp, dp, wd, dd, causal=True, workspace=ws)
    op_ref, lp_ref = OA.batch_prefill(wp, causal=True)
    od_ref, ld_ref = OA.batch_decode(wd)
    assert np.isnan(ld_ref).sum() == 4  # the 4 q heads of kv head 3 in decode request 1
    assert_parity_nan(op, lp, op_ref, lp_ref, "f16", f"pod prefill NaN code {kvd}")
    assert_parity_nan(od, ld, od_ref, ld_ref, "f16", f"pod decode NaN code {kvd}")


def test_pod_past_argument_capacities(gpu_device):
    """A prefill phase of 60 requests (more than the 48 whose geometry one
    launch's arguments carry: the prefill workgroups then read it from the
    device) with a decode phase of 300 requests (more than the 256 token
    prefix sums carried: every decode workgroup scans the page table itself),
    against the oracle."""
    say("pod past argument capacities")
    rng = np.random.default_rng(79)
    qo = rng.integers(1, 41, size=60)
    prefix = rng.integers(0, 101, size=60)
    dec = rng.integers(0, 201, size=300)
    wp = make_paged(79, qo_lens=list(qo), prefix_lens=list(prefix), hq=8, hkv=2, d=128, page=16, q="f16", kvd="e4m3",
                    extra_pages=2)
    wd = make_paged(80, kv_lens=list(dec), hq=8, hkv=2, d=128, page=16, q="f16", kvd="e4m3", extra_pages=2)
    dp, dd = upload(wp, gpu_device), upload(wd, gpu_device)
    (op, lp), (od, ld) = run_pod(wp, dp, wd, dd, causal=True)
    o_ref, l_ref = OA.batch_prefill(wp, causal=True)
    assert_parity(op, lp, o_ref, l_ref, "f16", "pod prefill phase, 60 requests")
    o_ref, l_ref = OA.batch_decode(wd)
    assert_parity(od, ld, o_ref, l_ref, "f16", "pod decode phase, 300 requests")

