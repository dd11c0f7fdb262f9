"""GPU parity tests for batched paged prefill with an fp8 query, through the
C ABI, against the float64 oracle.

The query arrives as fp8 codes with a per-tensor q_scale that joins k_scale
and sm_scale in the logit scale ("Enable Hopper FA3 FP8 attention in
decode.py", flashinfer PR #2148, review comments on q_scale); the output is
float16 or bfloat16.  S = Q K^T runs on the fp8 matrix cores with K kept in
fp8, P V in float16, so the tolerances are those of the 2-byte path.

With pv_fp8 the probabilities are rounded to e4m3 for P V on the fp8 MFMA
(the FA3 fp8 path of the pages).  Rounding to nearest with 3 mantissa bits
moves each probability p (relative to its row maximum) by at most 2^-4 p, or
2^-10 in the subnormal range, uniformly within that interval; the output,
normalised by the unrounded fp32 sum, then differs from the oracle by
sum_t e_t v_t / sum_t p_t.  The test bounds each element by 7 standard
deviations of that sum, sigma^2 = sum_t ((2^-4 p_t)^2 + 2^-20) / 3 * v_t^2 /
(sum_t p_t)^2, computed from the oracle's exact probabilities, plus the
output's own tolerance; the log-sum-exp (from the unrounded sum) keeps its
1e-3.  A zero query makes every probability exactly 1, so the output must be
the exact mean of the visible V rows: that pins the pairing of P and V keys.

Cases: both query formats against both cache formats, both output types,
head_dim 64 and 128, GQA groups 1 to 8, page sizes 1 to 128, causal and not,
ragged lengths that leave partial tiles; the causal-prefill workload (16 requests, qo 256..1024, prefix 0..2048, 32/8 heads, d 128)
with its query quantised to e4m3, at full size (whole requests and sampled
rows); requests without queries or keys; run-to-run and page-permutation
determinism (bitwise).
"""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from workloads import NAN_BITS, make_paged, make_workload
from gpu_util import LSE_TOL, O_TOL, T2, assert_parity, assert_parity_nan, paged_kv, plant_codes, say, upload
from attention_paged_fp8_amd import fi

pytestmark = pytest.mark.gpu


def run_fp8q(w: dict, d: dict, *, causal=True, kv=None, pv_fp8=False):
    T = int(w["qo_indptr"][-1])
    o = torch.full((T, w["num_qo_heads"], w["head_dim"]), float("nan"), dtype=T2[w["o_dtype"]], device=d["q"].device)
    lse = torch.full((T, w["num_qo_heads"]), float("nan"), dtype=torch.float32, device=d["q"].device)
    if kv is None:
        kv, keep = paged_kv(w, d)
    fi.fi_batch_prefill_paged_fp8q(d["q"], d["qo_indptr"], kv, o, q_dtype=w["q_dtype"], q_scale=w["q_scale"],
                                   causal=causal, pv_fp8=pv_fp8, lse=lse, qo_indptr_h=w["qo_indptr"])
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


SMALL = [
    # (q, kvd, o, page, d, hq, hkv, qo, prefix, causal)
    ("e4m3", "e4m3", "f16", 16, 128, 32, 8, (1, 37, 130, 64), (0, 100, 5, 300), True),
    ("e4m3", "e4m3", "bf16", 16, 128, 32, 8, (1, 37, 130, 64), (0, 100, 5, 300), False),
    ("e5m2", "e4m3", "f16", 64, 128, 16, 8, (200, 33), (70, 0), True),        # group 2
    ("e4m3", "e5m2", "bf16", 4, 64, 8, 8, (129, 3, 257), (1, 64, 0), True),   # group 1
    ("e5m2", "e5m2", "f16", 1, 64, 12, 4, (45, 90), (10, 0), True),           # group 3
    ("e4m3", "e5m2", "f16", 32, 128, 64, 8, (100, 65), (40, 1), True),        # group 8
    ("e5m2", "e4m3", "bf16", 128, 128, 32, 8, (70, 300), (400, 2), False),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"q{c[0]}-{c[1]}-o{c[2]}-p{c[3]}-d{c[4]}-h{c[5]}x{c[6]}-c{int(c[9])}" for c in SMALL])
def test_fp8q_small(gpu_device, case):
    q, kvd, o, page, d_, hq, hkv, qo, prefix, causal = case
    say("fp8q small", case)
    w = make_paged(91, qo_lens=list(qo), prefix_lens=list(prefix), hq=hq, hkv=hkv, d=d_, page=page, q=q, kvd=kvd,
                   o=o, extra_pages=2)
    dv = upload(w, gpu_device)
    og, lg = run_fp8q(w, dv, causal=causal)
    o_ref, l_ref = OA.batch_prefill(w, causal=causal)
    assert_parity(og, lg, o_ref, l_ref, o, str(case))


def _causal_prefill_fp8q():
    """The causal-prefill workload with its query quantised to e4m3
    (per-tensor scale): the same lengths, pages and draws."""
    return make_workload("causal_prefill", q="e4m3")


def test_causal_prefill_fp8q_full_size(gpu_device):
    say("causal_prefill fp8q")
    w = _causal_prefill_fp8q()
    d = upload(w, gpu_device)
    og, lg = run_fp8q(w, d)
    og2, lg2 = run_fp8q(w, d)
    assert np.array_equal(og, og2) and np.array_equal(lg, lg2), "fp8-query prefill is not deterministic"
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    err = assert_parity(og, lg, o_ref, l_ref, "f16", "causal-prefill workload, fp8 query")
    print(f"causal-prefill workload, fp8 query: max |o - oracle| = {err:.3e}")


@pytest.mark.parametrize("causal", [True, False])
def test_fp8q_requests_without_queries_or_keys(gpu_device, causal):
    say("fp8q empty requests", causal)
    w = make_paged(93, qo_lens=[0, 40, 13, 0, 7, 50], kv_lens=[5, 0, 200, 0, 7, 20], hq=8, hkv=2, d=64, page=16,
                   q="e5m2", kvd="e4m3", o="bf16")
    dv = upload(w, gpu_device)
    o, l = run_fp8q(w, dv, causal=causal)
    assert np.all(o[0:40] == 0) and np.all(np.isneginf(l[0:40]))
    o_ref, l_ref = OA.batch_prefill(w, causal=causal)
    assert_parity(o, l, o_ref, l_ref, "bf16", "fp8q empty requests")


def test_fp8q_page_permutation_bitwise(gpu_device):
    say("fp8q page permutation")
    w = make_paged(95, qo_lens=[300, 17, 129], prefix_lens=[700, 0, 63], hq=32, hkv=8, d=128, page=16, q="e4m3",
                   kvd="e4m3", o="f16", extra_pages=20)
    d = upload(w, gpu_device)
    o1, l1 = run_fp8q(w, d)
    P = w["k_pool"].shape[0]
    perm = np.random.default_rng(6).permutation(P)
    inv = np.argsort(perm)
    w2 = dict(w, k_pool=w["k_pool"][perm], v_pool=w["v_pool"][perm], indices=inv[w["indices"]].astype(np.int32))
    o2, l2 = run_fp8q(w2, upload(w2, gpu_device))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------------ fp8 P V
def pv8_sigma(w: dict, causal: bool) -> np.ndarray:
    """Per-element standard deviation of the e4m3 rounding of the
    probabilities, propagated to the output [tokens, H_qo, d] (see above)."""
    q_all = OA.query_values(w)
    hq, d = q_all.shape[1], q_all.shape[2]
    group = hq // w["num_kv_heads"]
    scale = OA.default_sm_scale(d)
    sig = np.zeros_like(q_all)
    qi = w["qo_indptr"]
    for i in range(len(qi) - 1):
        a, b = int(qi[i]), int(qi[i + 1])
        k, v = OA.paged_kv_values(w, i)
        n_q, n_kv = b - a, k.shape[0]
        if n_q == 0 or n_kv == 0:
            continue
        rows = np.arange(n_q)[:, None]
        cols = np.arange(n_kv)[None, :]
        allowed = (cols <= rows + (n_kv - n_q)) if causal else np.ones((n_q, n_kv), bool)
        for h in range(hq):
            g = h // group
            s_ = (q_all[a:b, h] @ k[:, g].T) * scale
            s_ = np.where(allowed, s_, -np.inf)
            m = s_.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            p_ = np.where(allowed, np.exp(s_ - m), 0.0)
            var = np.where(allowed, ((2.0 ** -4 * p_) ** 2 + 2.0 ** -20) / 3.0, 0.0)
            tot = p_.sum(axis=1, keepdims=True)
            tot = np.where(tot > 0, tot, 1.0)
            sig[a:b, h] = np.sqrt(var @ (v[:, g] ** 2)) / tot
    return sig


PV8 = [
    # (q, kvd, o, page, d, hq, hkv, qo, prefix, causal)
    ("e4m3", "e4m3", "f16", 16, 128, 32, 8, (1, 37, 130, 64), (0, 100, 5, 300), True),
    ("e5m2", "e4m3", "bf16", 16, 128, 16, 8, (200, 33), (70, 0), False),
    ("e4m3", "e5m2", "f16", 4, 64, 8, 8, (129, 3, 257), (1, 64, 0), True),
    ("e5m2", "e5m2", "bf16", 32, 128, 64, 8, (100, 65), (40, 1), True),
]


@pytest.mark.parametrize("case", PV8, ids=[f"q{c[0]}-{c[1]}-o{c[2]}-p{c[3]}-d{c[4]}-h{c[5]}x{c[6]}-c{int(c[9])}" for c in PV8])
def test_fp8q_pv8_small(gpu_device, case):
    q, kvd, o, page, d_, hq, hkv, qo, prefix, causal = case
    say("fp8q pv8", case)
    w = make_paged(97, qo_lens=list(qo), prefix_lens=list(prefix), hq=hq, hkv=hkv, d=d_, page=page, q=q, kvd=kvd,
                   o=o, extra_pages=2)
    dv = upload(w, gpu_device)
    og, lg = run_fp8q(w, dv, causal=causal, pv_fp8=True)
    o_ref, l_ref = OA.batch_prefill(w, causal=causal)
    assert np.all(np.isfinite(og)), "non-finite output"
    both_inf = np.isneginf(lg) & np.isneginf(l_ref)
    assert np.all(np.isfinite(lg[~both_inf])), "lse -inf mismatch"
    assert float(np.max(np.abs(lg[~both_inf] - l_ref[~both_inf]))) <= LSE_TOL
    bound = 7.0 * pv8_sigma(w, causal) + O_TOL[o]
    err = np.abs(og - o_ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"{case}: |o - oracle| = {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst}"
    # the rounding is visible but small: the mean error stays far below the bound
    assert float(err.mean()) < 0.25 * float(bound.mean())


@pytest.mark.parametrize("causal", [True, False])
def test_fp8q_pv8_zero_query_is_exact_mean(gpu_device, causal):
    say("fp8q pv8 zero query", causal)
    w = make_paged(98, qo_lens=[1, 37, 130, 64], prefix_lens=[0, 100, 5, 300], hq=16, hkv=8, d=128, page=16,
                   q="e4m3", kvd="e5m2", o="f16")
    w["q"][:] = 0
    dv = upload(w, gpu_device)
    og, lg = run_fp8q(w, dv, causal=causal, pv_fp8=True)
    o_ref, l_ref = OA.batch_prefill(w, causal=causal)
    assert_parity(og, lg, o_ref, l_ref, "f16", "zero query, fp8 P V")


def test_causal_prefill_fp8q_pv8_sampled_rows(gpu_device):
    """The causal-prefill workload, fp8 query, fp8 P V: sampled rows
    against the oracle within the rounding bound, lse at 1e-3."""
    say("causal_prefill fp8q pv8")
    w = _causal_prefill_fp8q()
    d = upload(w, gpu_device)
    og, lg = run_fp8q(w, d, pv_fp8=True)
    og2, lg2 = run_fp8q(w, d, pv_fp8=True)
    assert np.array_equal(og, og2) and np.array_equal(lg, lg2), "not deterministic"
    assert np.all(np.isfinite(og))
    i = 9
    a, b = int(w["qo_indptr"][i]), int(w["qo_indptr"][i + 1])
    sub = dict(w, qo_indptr=np.array([0, b - a], np.int32), q=w["q"][a:b], indptr=w["indptr"][i:i + 2] - w["indptr"][i],
               indices=w["indices"][w["indptr"][i]:w["indptr"][i + 1]], last_page_len=w["last_page_len"][i:i + 1])
    o_ref, l_ref = OA.batch_prefill(sub, causal=True)
    bound = 7.0 * pv8_sigma(sub, True) + O_TOL["f16"]
    err = np.abs(og[a:b] - o_ref)
    assert np.all(err <= bound), f"request {i}: max excess {float(np.max(err - bound)):.3e}"
    assert float(np.max(np.abs(lg[a:b] - l_ref))) <= LSE_TOL


@pytest.mark.parametrize("pv8", [False, True])
@pytest.mark.parametrize("q,kvd", [("e4m3", "e4m3"), ("e5m2", "e5m2")])
def test_ragged_and_single_fp8q_equal_paged(gpu_device, q, kvd, pv8):
    """fi_batch_prefill_ragged_fp8q over the same K/V values stored
    contiguously per request, and fi_single_prefill_fp8q on one request, give
    the bits of fi_batch_prefill_paged_fp8q (the same kernel, addressing rows
    instead of pages); the 16-bit P V mode also against the oracle."""
    say("ragged/single fp8q", q, kvd, pv8)
    from workloads import ragged_rows
    w = make_paged(61, qo_lens=[1, 70, 300, 129], prefix_lens=[0, 45, 600, 3], hq=32, hkv=8, d=128, page=16, q=q,
                   kvd=kvd, o="f16")
    d = upload(w, gpu_device)
    op, lp = run_fp8q(w, d, causal=True, pv_fp8=pv8)
    if not pv8:
        o_ref, l_ref = OA.batch_prefill(w, causal=True)
        assert_parity(op, lp, o_ref, l_ref, "f16", "paged fp8q")
    kr, vr, indptr = ragged_rows(w, lead=3, tail=2)
    kt, vt = torch.from_numpy(kr).to(gpu_device), torch.from_numpy(vr).to(gpu_device)
    ind = torch.from_numpy(indptr).to(gpu_device)
    kv, keep = fi.make_ragged_kv(kt, vt, ind, k_scale=w["k_scale"], v_scale=w["v_scale"], kv_dtype=kvd, indptr_h=indptr)
    T, H, D = int(w["qo_indptr"][-1]), w["num_qo_heads"], w["head_dim"]
    o = torch.full((T, H, D), float("nan"), dtype=torch.float16, device=gpu_device)
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device=gpu_device)
    fi.fi_batch_prefill_ragged_fp8q(d["q"], d["qo_indptr"], kv, o, q_dtype=q, q_scale=w["q_scale"], causal=True,
                                    pv_fp8=pv8, lse=lse, qo_indptr_h=w["qo_indptr"])
    torch.cuda.synchronize()
    assert np.array_equal(o.double().cpu().numpy(), op) and np.array_equal(lse.double().cpu().numpy(), lp)
    # one request (the third) through the single call
    i = 2
    q0, q1 = int(w["qo_indptr"][i]), int(w["qo_indptr"][i + 1])
    a, e = int(indptr[i]), int(indptr[i + 1])
    ks, vs = kt[a:e].contiguous(), vt[a:e].contiguous()
    o1 = torch.full((q1 - q0, H, D), float("nan"), dtype=torch.float16, device=gpu_device)
    l1 = torch.full((q1 - q0, H), float("nan"), dtype=torch.float32, device=gpu_device)
    fi.fi_single_prefill_fp8q(d["q"][q0:q1].contiguous(), ks, vs, o1, q_dtype=q, q_scale=w["q_scale"], causal=True,
                              pv_fp8=pv8, k_scale=w["k_scale"], v_scale=w["v_scale"], kv_dtype=kvd, lse=l1)
    torch.cuda.synchronize()
    assert np.array_equal(o1.double().cpu().numpy(), op[q0:q1]) and np.array_equal(l1.double().cpu().numpy(), lp[q0:q1])


@pytest.mark.parametrize("pv_fp8", [False, True])
@pytest.mark.parametrize("kvd", ["e4m3", "e5m2"])
def test_fp8q_nan_code_propagates(gpu_device, kvd, pv_fp8):
    """The cache format's NaN code in one K element of a key only the later
    rows see and in one V element of a prefix key every row sees, with the
    raw codes on the fp8 matrix cores: exactly the oracle's NaN outputs are
    NaN (whole rows from the first row that sees the K code, the V code's
    column of every row).  With P V in f16 every other output matches the
    oracle to the usual tolerance; with fp8 P V they are finite (their
    values are held to the derived bound by the other tests)."""
    say("fp8q NaN code", kvd, pv_fp8)
    w = make_paged(38, qo_lens=[40, 130, 64], prefix_lens=[10, 300, 0], hq=32, hkv=8, d=128, page=16, q="e4m3",
                   kvd=kvd, o="f16", extra_pages=2)
    plant_codes(w, 1, [("k_pool", 350, 5, 17, NAN_BITS[kvd]), ("v_pool", 100, 2, 40, NAN_BITS[kvd])])
    dv = upload(w, gpu_device)
    og, lg = run_fp8q(w, dv, causal=True, pv_fp8=pv_fp8)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    assert np.isnan(l_ref).sum() == (130 - 50) * 4
    if not pv_fp8:
        assert_parity_nan(og, lg, o_ref, l_ref, "f16", f"fp8q NaN code {kvd}")
        return
    assert np.array_equal(np.isnan(og), np.isnan(o_ref)) and np.array_equal(np.isnan(lg), np.isnan(l_ref))
    assert np.isfinite(og[~np.isnan(o_ref)]).all()

