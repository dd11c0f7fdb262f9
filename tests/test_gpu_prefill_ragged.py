"""GPU parity tests for prefill over a ragged (non-paged) K/V and for the
single-request prefill, through the C ABI, against the float64 oracle.

The ragged and single calls are the batch-prefill and single-prefill run
entry points of "fp8 KV cache in the in-tree prefill kernel"
(AMD-Ecosystem/flashinfer PR #368, Architecture / design notes); its Test
plan holds fp8 to the dequantized run bitwise across single, paged and ragged
layouts.  Here:

* ragged K/V built from a paged workload (the same stored elements, each
  request's tokens contiguous, poisoned rows before the first request and
  after the last) against the oracle, and bitwise against the paged call;
* fp8 ragged K/V against the same values pre-widened to q's type, bitwise;
* single-request prefill against the oracle and bitwise against that request
  inside a paged batch, including a request without keys;
* ragged requests without queries or keys, and rows that see no key;
* the causal-prefill workload (16 requests, qo 256..1024, prefix 0..2048, 32/8 heads, d 128) as a ragged batch, bitwise against the
  paged call at full size.
"""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from oracle.fp8 import fp8_table
from workloads import make_paged, make_workload, ragged_rows
from gpu_util import T2, assert_parity, dev_pool, run_prefill, say, upload
from attention_paged_fp8_amd import fi

pytestmark = pytest.mark.gpu

CASES = [
    # (kvd, q, o, d, hq, hkv, qo, prefix, causal)
    ("e4m3", "f16", "f16", 128, 32, 8, (1, 37, 130, 64), (0, 100, 5, 300), True),
    ("e5m2", "bf16", "bf16", 128, 16, 8, (200, 33), (70, 0), False),
    ("e4m3", "bf16", "f16", 64, 8, 8, (129, 3, 257), (1, 64, 0), True),
    ("e5m2", "f16", "bf16", 64, 12, 4, (45, 90), (10, 0), True),
    ("f16", "f16", "f16", 128, 32, 8, (77, 256), (3, 128), True),
    ("bf16", "bf16", "bf16", 64, 4, 2, (150,), (200,), False),
    ("e4m3fnuz", "bf16", "bf16", 128, 32, 8, (1, 37, 130), (0, 100, 5), True),
    ("e5m2fnuz", "f16", "f16", 64, 8, 2, (129, 3), (1, 64), False),
]


def ragged_kv(w: dict, device, lead=0, tail=0, kv_dtype=None, k=None, v=None):
    kr, vr, indptr = ragged_rows(w, lead=lead, tail=tail)
    kd = kv_dtype or w["kv_dtype"]
    kt = dev_pool(kr, w["kv_dtype"], device) if k is None else k
    vt = dev_pool(vr, w["kv_dtype"], device) if v is None else v
    ind = torch.from_numpy(indptr).to(device)
    kv, keep = fi.make_ragged_kv(kt, vt, ind, k_scale=w["k_scale"], v_scale=w["v_scale"], kv_dtype=kd,
                                 indptr_h=indptr)
    return kv, (keep, kt, vt, ind, kr, vr)


def run_ragged(w: dict, d: dict, kv, *, causal=True):
    T = int(w["qo_indptr"][-1])
    o = torch.full((T, w["num_qo_heads"], w["head_dim"]), float("nan"), dtype=T2[w["o_dtype"]], device=d["q"].device)
    lse = torch.full((T, w["num_qo_heads"]), float("nan"), dtype=torch.float32, device=d["q"].device)
    fi.fi_batch_prefill_ragged(d["q"], d["qo_indptr"], kv, o, causal=causal, lse=lse, qo_indptr_h=w["qo_indptr"])
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-q{c[1]}-o{c[2]}-d{c[3]}-h{c[4]}x{c[5]}-c{int(c[8])}" for c in CASES])
def test_ragged_small(gpu_device, case):
    kvd, q, o, d_, hq, hkv, qo, prefix, causal = case
    say("ragged small", case)
    w = make_paged(71, qo_lens=list(qo), prefix_lens=list(prefix), hq=hq, hkv=hkv, d=d_, page=16, q=q, kvd=kvd, o=o)
    dv = upload(w, gpu_device)
    kv, keep = ragged_kv(w, gpu_device, lead=5, tail=7)
    og, lg = run_ragged(w, dv, kv, causal=causal)
    o_ref, l_ref = OA.batch_prefill(w, causal=causal)
    assert_parity(og, lg, o_ref, l_ref, o, str(case))
    op, lp, _ = run_prefill(w, dv, causal=causal)
    assert np.array_equal(og, op) and np.array_equal(lg, lp), "ragged and paged calls differ"


@pytest.mark.parametrize("kvd,q", [("e4m3", "f16"), ("e5m2", "bf16")])
def test_ragged_fp8_equals_prewidened_bitwise(gpu_device, kvd, q):
    say("ragged prewidened", kvd, q)
    w = make_paged(73, qo_lens=[300, 17, 129], prefix_lens=[700, 0, 63], hq=32, hkv=8, d=128, page=16, q=q, kvd=kvd)
    dv = upload(w, gpu_device)
    kv1, keep1 = ragged_kv(w, gpu_device, lead=3)
    o1, l1 = run_ragged(w, dv, kv1)
    kr, vr = keep1[4], keep1[5]
    tab = fp8_table(kvd)
    k2 = torch.from_numpy(tab[kr].astype(np.float32)).to(T2[q]).to(gpu_device)
    v2 = torch.from_numpy(tab[vr].astype(np.float32)).to(T2[q]).to(gpu_device)
    kv2, keep2 = ragged_kv(w, gpu_device, lead=3, kv_dtype=q, k=k2, v=v2)
    o2, l2 = run_ragged(w, dv, kv2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [True, False])
def test_ragged_requests_without_queries_or_keys(gpu_device, causal):
    """qo_len 0 writes nothing; kv_len 0 gives o = 0 and lse = -inf; under the
    causal mask the first qo_len - kv_len rows of a short-KV request see nothing."""
    say("ragged empty requests", causal)
    w = make_paged(75, qo_lens=[0, 40, 13, 0, 7, 50], kv_lens=[5, 0, 200, 0, 7, 20], hq=8, hkv=2, d=64, page=16,
                   q="bf16", kvd="e5m2")
    dv = upload(w, gpu_device)
    kv, keep = ragged_kv(w, gpu_device, lead=1, tail=2)
    o, l = run_ragged(w, dv, kv, causal=causal)
    assert np.all(o[0:40] == 0) and np.all(np.isneginf(l[0:40]))
    o_ref, l_ref = OA.batch_prefill(w, causal=causal)
    assert_parity(o, l, o_ref, l_ref, "bf16", "ragged empty requests")


SINGLE = [
    # (kvd, q, d, hq, hkv, qo, kv, causal)
    ("e4m3", "f16", 128, 32, 8, 300, 1000, True),
    ("e5m2", "bf16", 128, 32, 8, 1, 517, True),
    ("e4m3", "bf16", 64, 4, 4, 130, 130, False),
    ("f16", "f16", 64, 12, 4, 77, 40, True),    # kv shorter than qo: early rows see nothing
    ("e4m3", "f16", 128, 16, 8, 64, 0, True),   # no keys
    ("e4m3fnuz", "f16", 128, 32, 8, 200, 700, True),
]


@pytest.mark.parametrize("case", SINGLE, ids=[f"{c[0]}-q{c[1]}-d{c[2]}-h{c[3]}x{c[4]}-qo{c[5]}-kv{c[6]}-c{int(c[7])}" for c in SINGLE])
def test_single_prefill(gpu_device, case):
    kvd, q, d_, hq, hkv, qo, kvl, causal = case
    say("single prefill", case)
    w = make_paged(77, qo_lens=[qo], kv_lens=[kvl], hq=hq, hkv=hkv, d=d_, page=16, q=q, kvd=kvd)
    dv = upload(w, gpu_device)
    kr, vr, _ = ragged_rows(w)
    k = dev_pool(kr, kvd, gpu_device)
    v = dev_pool(vr, kvd, gpu_device)
    o = torch.full((qo, hq, d_), float("nan"), dtype=T2[q], device=gpu_device)
    lse = torch.full((qo, hq), float("nan"), dtype=torch.float32, device=gpu_device)
    fi.fi_single_prefill(dv["q"], k, v, o, causal=causal, k_scale=w["k_scale"], v_scale=w["v_scale"], kv_dtype=kvd,
                         lse=lse)
    torch.cuda.synchronize()
    og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
    o_ref, l_ref = OA.batch_prefill(w, causal=causal)
    assert_parity(og, lg, o_ref, l_ref, q, str(case))
    if kvl == 0:  # an empty pool has no strides to describe a paged cache with
        assert np.all(og == 0) and np.all(np.isneginf(lg))
        return
    op, lp, _ = run_prefill(w, dv, causal=causal)
    assert np.array_equal(og, op) and np.array_equal(lg, lp), "single and paged calls differ"


def test_causal_prefill_ragged_equals_paged(gpu_device):
    """The causal-prefill workload as a ragged batch: bitwise equal to
    the paged call, which the paged tests hold to the oracle."""
    say("causal_prefill ragged")
    w = make_workload("causal_prefill")
    dv = upload(w, gpu_device)
    kv, keep = ragged_kv(w, gpu_device, lead=16)
    og, lg = run_ragged(w, dv, kv)
    op, lp, _ = run_prefill(w, dv, causal=True)
    assert np.array_equal(og, op) and np.array_equal(lg, lp)
    i = 3
    a, b = int(w["qo_indptr"][i]), int(w["qo_indptr"][i + 1])
    o_ref, l_ref = OA.batch_prefill(w, causal=True, requests=[i])
    assert_parity(og[a:b], lg[a:b], o_ref[a:b], l_ref[a:b], "f16", "causal-prefill workload ragged request 3")
