"""GPU parity tests for batched paged prefill (causal and not), through the C
ABI, against the float64 oracle.

Cases: the causal prefill configuration (3) at full size -- four requests
compared element by element and sampled rows of every request; a matrix of
small shapes (GQA groups 1, 2, 3, 4, 8; head_dim 64 and 128; page sizes 1 to
64; fp8 and same-type 2-byte KV; causal and non-causal; ragged query and
prefix lengths that leave partial tiles); rows with no visible key; decode
equal to prefill with one query per request; run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from workloads import make_config, make_paged
from gpu_util import assert_parity, run_decode, run_prefill, say, upload

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


def test_config3_full_size(gpu_device):
    say("config3")
    w = make_config(3)
    d = upload(w, gpu_device)
    og, lg, _ = run_prefill(w, d, causal=True)
    og2, lg2, _ = run_prefill(w, d, causal=True)
    assert np.array_equal(og, og2) and np.array_equal(lg, lg2), "prefill is not deterministic"
    reqs = [0, 5, 10, 15]
    o_ref, l_ref = OA.batch_prefill(w, causal=True, requests=reqs)
    qi = w["qo_indptr"]
    for i in reqs:
        a, b = int(qi[i]), int(qi[i + 1])
        assert_parity(og[a:b], lg[a:b], o_ref[a:b], l_ref[a:b], "f16", f"config 3 request {i}")
    # sampled rows of every request: first, last and random rows, every head
    rng = np.random.default_rng(0)
    toks, heads = [], []
    for i in range(len(w["qo_lens"])):
        a, b = int(qi[i]), int(qi[i + 1])
        for t in {a, b - 1, int(rng.integers(a, b)), int(rng.integers(a, b))}:
            for h in rng.choice(32, 4, replace=False):
                toks.append(t)
                heads.append(int(h))
    o_s, l_s = OA.attention_rows(w, toks, heads, causal=True)
    assert_parity(og[toks, heads], lg[toks, heads], o_s, l_s, "f16", "config 3 sampled rows")


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
