"""Pins for the oracle's attention and merge (CPU only).

Each pin is a function of the oracle module, so the same pins also run against
copies of the oracle with a planted mistake (test_planted_mistakes_are_caught):
a dropped term, a wrong sign or index, an off-by-one mask, a transposed
operand.  Every planted mistake must fail at least one pin.

Pins, and what fixes them independently of the oracle's own code:
  * brute force: scalar loops that walk the page table slot by slot, decode
    elements with torch's casts, and normalise exp(s) directly, on tiny inputs;
  * closed forms: one key gives o = V0 and lse = s0; q = 0 gives the mean of V
    and lse = ln(n); constant V gives V; identical keys give uniform weights;
  * invariants: softmax weights sum to one (V = 1 gives 1), the result does
    not depend on where pages sit in the pool, decode equals prefill with one
    query, split-and-merge equals the unsplit result, GQA equals MHA with
    repeated kv heads, and scaling k_scale by c equals scaling sm_scale by c
    (the fold recorded in "fp8 KV cache in the in-tree prefill kernel",
    Test plan, k_scale/v_scale item); the same for q_scale of an fp8 query;
  * causal: with no prefix, query row 0 sees only key 0 and the last row sees
    every key;
  * a NaN stored in K poisons exactly the rows that read it, and a NaN or inf
    stored in V only the rows that see its key, in its own column (brute
    force, which skips hidden keys); the contiguous single-decode form equals
    the scalar loops.
"""
import importlib.util
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

import oracle.attention as A
from workloads import make_paged

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_TDT = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2,
        "e4m3fnuz": torch.float8_e4m3fnuz, "e5m2fnuz": torch.float8_e5m2fnuz}


def _torch_decode(raw, dtype):
    """Independent element decode through torch's casts."""
    t = torch.from_numpy(np.ascontiguousarray(raw))
    if dtype in ("f16", "bf16"):
        t = t.view(torch.int16)
    return t.view(_TDT[dtype]).to(torch.float64).numpy()


def brute_force(w, causal, sm_scale=None):
    """Scalar-loop definition: page walk slot by slot, exp without a max
    shift (inputs are tiny and logits small), explicit sums."""
    q = _torch_decode(w["q"], w["q_dtype"]) * w.get("q_scale", 1.0)
    hq, d = q.shape[1], q.shape[2]
    hkv = w["k_pool"].shape[2]
    grp = hq // hkv
    scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    o = np.zeros_like(q)
    lse = np.full(q.shape[:2], -np.inf)
    B = len(w["indptr"]) - 1
    for i in range(B):
        keys, vals = [], []
        pages = list(w["indices"][w["indptr"][i]:w["indptr"][i + 1]])
        for j, pg in enumerate(pages):
            nslot = w["page_size"] if j < len(pages) - 1 else int(w["last_page_len"][i])
            for s in range(nslot):
                keys.append(_torch_decode(w["k_pool"][pg, s], w["kv_dtype"]) * w["k_scale"])
                vals.append(_torch_decode(w["v_pool"][pg, s], w["kv_dtype"]) * w["v_scale"])
        n_kv = len(keys)
        a, b = int(w["qo_indptr"][i]), int(w["qo_indptr"][i + 1])
        n_q = b - a
        for r in range(n_q):
            for h in range(hq):
                g = h // grp
                ws, acc, seen = 0.0, np.zeros(d), 0
                for t in range(n_kv):
                    if causal and t > r + n_kv - n_q:
                        continue
                    seen += 1
                    s = 0.0
                    for c in range(d):
                        s += q[a + r, h, c] * keys[t][g, c]
                    e = math.exp(s * scale)
                    ws += e
                    acc = acc + e * vals[t][g]
                if seen > 0:  # a NaN logit makes ws NaN, and o and lse with it
                    o[a + r, h] = acc / ws
                    lse[a + r, h] = math.log(ws) if ws == ws else math.nan
    return o, lse


def _tiny_decode(seed=0, kvd="e4m3", q="f16", page=4, hq=4, hkv=2, d=8, lens=(1, 7, 13, 4)):
    return make_paged(seed, kv_lens=list(lens), hq=hq, hkv=hkv, d=d, page=page, q=q, kvd=kvd)


def _tiny_prefill(seed=1, kvd="e5m2", q="bf16", page=4, hq=4, hkv=2, d=8, qo=(1, 3, 5), prefix=(0, 2, 6)):
    return make_paged(seed, qo_lens=list(qo), prefix_lens=list(prefix), hq=hq, hkv=hkv, d=d, page=page, q=q, kvd=kvd)


# ---------------------------------------------------------------- pins
def pin_brute_force_decode(M):
    for seed, kvd, q, page in ((0, "e4m3", "f16", 4), (3, "e5m2", "bf16", 16), (4, "bf16", "f16", 4)):
        w = _tiny_decode(seed, kvd, q, page)
        o, l = M.batch_decode(w)
        ob, lb = brute_force(w, causal=False)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


def pin_brute_force_prefill(M):
    for seed, page in ((1, 4), (2, 16)):
        w = _tiny_prefill(seed, page=page)
        o, l = M.batch_prefill(w, causal=True)
        ob, lb = brute_force(w, causal=True)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)
        o, l = M.batch_prefill(w, causal=False)
        ob, lb = brute_force(w, causal=False)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)


def pin_closed_forms(M):
    rng = np.random.default_rng(7)
    d = 6
    # one key: o = V0, lse = s0
    q = rng.standard_normal((1, 2, d)); k = rng.standard_normal((1, 1, d)); v = rng.standard_normal((1, 1, d))
    o, l = M.attention(q, k, v, causal=False, sm_scale=0.3)
    np.testing.assert_allclose(o[0, 0], v[0, 0], atol=1e-15)
    np.testing.assert_allclose(l[0], 0.3 * q[0] @ k[0, 0], atol=1e-14)
    # q = 0: uniform weights, lse = ln n
    n = 9
    k = rng.standard_normal((n, 1, d)); v = rng.standard_normal((n, 1, d))
    o, l = M.attention(np.zeros((1, 1, d)), k, v, causal=False, sm_scale=0.5)
    np.testing.assert_allclose(o[0, 0], v[:, 0].mean(0), atol=1e-14)
    np.testing.assert_allclose(l[0, 0], math.log(n), atol=1e-14)
    # constant V gives V
    q = rng.standard_normal((3, 2, d)); vc = np.tile(rng.standard_normal(d), (n, 1, 1))
    o, _ = M.attention(q, k, vc, causal=False, sm_scale=1.0)
    np.testing.assert_allclose(o, np.broadcast_to(vc[0, 0], o.shape), atol=1e-14)
    # identical keys: uniform weights, lse = s + ln n
    kk = np.tile(rng.standard_normal(d), (n, 1, 1))
    o, l = M.attention(q, kk, v, causal=False, sm_scale=0.7)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, 0].mean(0), o.shape), atol=1e-14)
    np.testing.assert_allclose(l, 0.7 * (q @ kk[0, 0]) + math.log(n), atol=1e-13)


def pin_weights_sum_to_one(M):
    rng = np.random.default_rng(11)
    q = rng.standard_normal((5, 4, 8)) * 3
    k = rng.standard_normal((17, 2, 8)) * 3
    o, _ = M.attention(q, k, np.ones((17, 2, 8)), causal=True, sm_scale=0.4)
    np.testing.assert_allclose(o, 1.0, atol=1e-13)


def pin_page_permutation(M):
    w = _tiny_decode(5, lens=(9, 1, 12))
    o1, l1 = M.batch_decode(w)
    P = w["k_pool"].shape[0]
    perm = np.random.default_rng(0).permutation(P)  # new position of old page p: inv
    w2 = dict(w)
    w2["k_pool"] = w["k_pool"][perm]
    w2["v_pool"] = w["v_pool"][perm]
    inv = np.argsort(perm)
    w2["indices"] = inv[w["indices"]].astype(np.int32)
    o2, l2 = M.batch_decode(w2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_decode_equals_prefill_one_query(M):
    w = _tiny_decode(6)
    o1, l1 = M.batch_decode(w)
    o2, l2 = M.batch_prefill(w, causal=True)
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    np.testing.assert_allclose(l1, l2, atol=1e-15)


def pin_split_merge(M):
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 4, 8)); k = rng.standard_normal((30, 2, 8)); v = rng.standard_normal((30, 2, 8))
    o, l = M.attention(q, k, v, causal=False, sm_scale=0.35)
    cuts = [0, 4, 4, 19, 30]  # includes an empty chunk
    parts = [M.attention(q, k[a:b], v[a:b], causal=False, sm_scale=0.35) for a, b in zip(cuts[:-1], cuts[1:])]
    om, lm = M.merge_states(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, l, atol=1e-13)
    # all chunks empty -> 0 / -inf
    oe, le = M.merge_states(np.zeros((2, 1, 4, 8)), np.full((2, 1, 4), -np.inf))
    assert np.all(oe == 0) and np.all(np.isneginf(le))


def pin_gqa_equals_repeated_mha(M):
    rng = np.random.default_rng(13)
    q = rng.standard_normal((3, 6, 8)); k = rng.standard_normal((11, 2, 8)); v = rng.standard_normal((11, 2, 8))
    o, l = M.attention(q, k, v, causal=True, sm_scale=0.3)
    kr = np.repeat(k, 3, axis=1); vr = np.repeat(v, 3, axis=1)
    o2, l2 = M.attention(q, kr, vr, causal=True, sm_scale=0.3)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(l, l2, atol=1e-14)
    # and each head separately equals attention with its own kv head
    for h in range(6):
        oh, lh = M.attention(q[:, h:h + 1], k[:, h // 3:h // 3 + 1], v[:, h // 3:h // 3 + 1], causal=True, sm_scale=0.3)
        np.testing.assert_allclose(o[:, h:h + 1], oh, atol=1e-14)


def pin_kscale_fold(M):
    w = _tiny_decode(8)
    c = 3.0
    w2 = dict(w); w2["k_scale"] = w["k_scale"] * c
    o1, l1 = M.batch_decode(w2, sm_scale=0.25)
    o2, l2 = M.batch_decode(w, sm_scale=0.25 * c)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-12)
    # v_scale is linear on the output
    w3 = dict(w); w3["v_scale"] = w["v_scale"] * c
    o3, _ = M.batch_decode(w3, sm_scale=0.25)
    o4, _ = M.batch_decode(w, sm_scale=0.25)
    np.testing.assert_allclose(o3, c * o4, atol=1e-13)


def pin_fp8_query(M):
    """An fp8 query with its per-tensor q_scale: brute force on tiny inputs,
    and scaling q_scale by c equals scaling sm_scale by c (the fold of
    "Enable Hopper FA3 FP8 attention in decode.py", flashinfer PR #2148,
    review comments on q_scale)."""
    for seed, q, kvd in ((11, "e4m3", "e4m3"), (12, "e5m2", "e4m3"), (13, "e4m3", "e5m2")):
        w = make_paged(seed, qo_lens=[1, 3, 5], prefix_lens=[0, 2, 6], hq=4, hkv=2, d=8, page=4, q=q, kvd=kvd, o="f16")
        assert w["q_scale"] != 1.0
        o, l = M.batch_prefill(w, causal=True)
        ob, lb = brute_force(w, causal=True)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)
    c = 2.5
    w2 = dict(w); w2["q_scale"] = w["q_scale"] * c
    o1, l1 = M.batch_prefill(w2, causal=True, sm_scale=0.3)
    o2, l2 = M.batch_prefill(w, causal=True, sm_scale=0.3 * c)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def pin_causal_rows(M):
    rng = np.random.default_rng(14)
    q = rng.standard_normal((6, 2, 4)); k = rng.standard_normal((6, 1, 4)); v = rng.standard_normal((6, 1, 4))
    o, l = M.attention(q, k, v, causal=True, sm_scale=1.0)
    np.testing.assert_allclose(o[0, :], np.broadcast_to(v[0, 0], (2, 4)), atol=1e-15)
    onc, _ = M.attention(q, k, v, causal=False, sm_scale=1.0)
    np.testing.assert_allclose(o[-1], onc[-1], atol=1e-15)
    # with a prefix of 2 keys, row 0 sees keys 0..2
    k8 = rng.standard_normal((8, 1, 4)); v8 = rng.standard_normal((8, 1, 4))
    o8, _ = M.attention(q, k8, v8, causal=True, sm_scale=1.0)
    o3, _ = M.attention(q[:1], k8[:3], v8[:3], causal=False, sm_scale=1.0)
    np.testing.assert_allclose(o8[:1], o3, atol=1e-15)


def pin_sampled_rows(M):
    w = _tiny_prefill(9)
    o, l = M.batch_prefill(w, causal=True)
    toks = list(range(o.shape[0]))
    heads = [t % 4 for t in toks]
    os_, ls_ = M.attention_rows(w, toks, heads, causal=True)
    for n, (t, h) in enumerate(zip(toks, heads)):
        np.testing.assert_allclose(os_[n], o[t, h], atol=1e-14)
        np.testing.assert_allclose(ls_[n], l[t, h], atol=1e-14)


def pin_empty_request(M):
    w = _tiny_decode(10, lens=(5, 0, 3))
    o, l = M.batch_decode(w)
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))
    ob, lb = brute_force(w, causal=False)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(l[[0, 2]], lb[[0, 2]], atol=1e-12)


def pin_nan_propagates(M):
    """A NaN code in one K element of one request and kv head: the q heads of
    that kv head in that request come out NaN (brute force: exp(NaN) poisons
    the sums), every other output is unchanged; an empty row stays o = 0,
    lse = -inf."""
    w = _tiny_decode(11, kvd="e4m3", lens=(5, 9, 3))
    i, g = 1, 1
    pg = w["indices"][w["indptr"][i]]
    w["k_pool"][pg, 2, g, 3] = 0x7F  # OCP e4m3 NaN
    o, l = M.batch_decode(w)
    ob, lb = brute_force(w, causal=False)
    bad = np.zeros(o.shape[:2], dtype=bool)
    bad[i, 2 * g:2 * g + 2] = True  # 4 q heads over 2 kv heads
    assert np.isnan(ob[bad]).all() and np.isnan(lb[bad]).all()
    assert np.isnan(o[bad]).all() and np.isnan(l[bad]).all()
    np.testing.assert_allclose(o[~bad], ob[~bad], atol=1e-12)
    np.testing.assert_allclose(l[~bad], lb[~bad], atol=1e-12)
    # merge: a NaN partial state poisons the merged one, an empty one does not
    om, lm = M.merge_states(np.array([[[1.0, 2.0]], [[3.0, 4.0]]]), np.array([[np.nan], [0.5]]))
    assert np.isnan(om).all() and np.isnan(lm).all()
    om, lm = M.merge_states(np.array([[[1.0, 2.0]], [[3.0, 4.0]]]), np.array([[-np.inf], [0.5]]))
    np.testing.assert_allclose(om[0], [3.0, 4.0], atol=1e-15)


def pin_masked_nonfinite_v(M):
    """A NaN and an inf stored in V under a causal mask reach, in their own
    column, exactly the rows that see their key (brute force skips hidden
    keys): rows the mask hides the key from stay finite, and so does every
    LSE."""
    w = _tiny_prefill(5, kvd="e5m2", qo=(1, 3, 5), prefix=(0, 2, 6))
    i, ps = 2, w["page_size"]
    n_kv = 11  # 5 queries after a prefix of 6: row r sees keys t <= r + 6
    assert A.kv_len_of(w["indptr"], w["last_page_len"], ps, i) == n_kv
    for t, g, c, code in ((8, 1, 3, 0x7F), (9, 0, 5, 0x7C)):  # e5m2 NaN, +inf
        w["v_pool"][w["indices"][w["indptr"][i] + t // ps], t % ps, g, c] = code
    o, l = M.batch_prefill(w, causal=True)
    ob, lb = brute_force(w, causal=True)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)
    a = int(w["qo_indptr"][i])
    assert np.isfinite(l).all()
    assert np.isfinite(o[a:a + 2, 2:4, 3]).all() and np.isnan(o[a + 2:a + 5, 2:4, 3]).all()
    assert np.isfinite(o[a:a + 3, 0:2, 5]).all() and np.isposinf(o[a + 3:a + 5, 0:2, 5]).all()
    o[a + 2:a + 5, 2:4, 3] = 0.0
    o[a + 3:a + 5, 0:2, 5] = 0.0
    assert np.isfinite(o).all()


def pin_single_decode(M):
    """single_decode on contiguous K/V rows against the scalar-loop definition
    of a one-request paged workload holding the same rows (pages contiguous)."""
    for seed, kvd, q in ((12, "e4m3", "f16"), (13, "e5m2fnuz", "bf16"), (14, "bf16", "f16")):
        w = make_paged(seed, kv_lens=[11], hq=4, hkv=2, d=8, page=4, q=q, kvd=kvd, contiguous=True)
        n = int(w["kv_lens"][0])
        k = w["k_pool"].reshape(-1, 2, 8)[:n]
        v = w["v_pool"].reshape(-1, 2, 8)[:n]
        o, l = M.single_decode(w["q"][0], q, k, v, kvd, w["k_scale"], w["v_scale"])
        ob, lb = brute_force(w, causal=False)
        np.testing.assert_allclose(o, ob[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, lb[0], rtol=0, atol=1e-12)


PINS = [pin_empty_request, pin_nan_propagates, pin_masked_nonfinite_v, pin_single_decode, pin_brute_force_decode, pin_brute_force_prefill, pin_closed_forms, pin_weights_sum_to_one,
        pin_page_permutation, pin_decode_equals_prefill_one_query, pin_split_merge,
        pin_gqa_equals_repeated_mha, pin_kscale_fold, pin_fp8_query, pin_causal_rows, pin_sampled_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(A)


# ---------------------------------------------------------------- planted mistakes
MUTATIONS = {
    "gqa_modulo_mapping": ("qg = q[:, g * group:(g + 1) * group, :]", "qg = q[:, g::h_kv, :]"),
    "causal_off_by_one": ("allowed = cols <= rows + (n_kv - n_q)", "allowed = cols < rows + (n_kv - n_q)"),
    "causal_not_end_aligned": ("allowed = cols <= rows + (n_kv - n_q)", "allowed = cols <= rows"),
    "dropped_sm_scale": ("s = (qg.reshape(n_q * group, d) @ kg.T) * sm_scale", "s = (qg.reshape(n_q * group, d) @ kg.T)"),
    "no_max_in_lse": ("m[..., 0] + np.log(", "np.log("),
    "wrong_sign_exp": ("p = np.exp(s - m_safe)", "p = np.exp(m_safe - s)"),
    "v_scale_dropped": ('v = decode_elements(v_raw, w["kv_dtype"]) * float(w["v_scale"])', 'v = decode_elements(v_raw, w["kv_dtype"])'),
    "k_scale_on_v": ('k = decode_elements(k_raw, w["kv_dtype"]) * float(w["k_scale"])', 'k = decode_elements(k_raw, w["kv_dtype"]) * float(w["v_scale"])'),
    "last_page_off_by_one": ("return (npages - 1) * page_size + int(last_page_len[i])", "return (npages - 1) * page_size + int(last_page_len[i]) - 1"),
    "slot_uses_page_index": ("slots = t % page_size", "slots = (t // page_size) % page_size"),
    "merge_unweighted": ("o = (coef[..., None] * o_parts).sum(axis=0)", "o = o_parts.mean(axis=0)"),
    "transposed_pv": ("@ np.where(vfin, vg, 0.0))", "@ np.where(vfin, vg, 0.0)[::-1])"),
    "masked_v_leaks": ("@ np.where(vfin, vg, 0.0))", "@ vg)"),
    "default_scale_wrong": ("return 1.0 / math.sqrt(head_dim)", "return 1.0 / head_dim"),
    "nan_as_empty_row": ("has = np.broadcast_to(allowed.any(axis=-1)[:, None, None], m.shape)", "has = np.isfinite(m)"),
    "single_v_scale_dropped": ("v = decode_elements(v_raw, kv_dtype) * float(v_scale)", "v = decode_elements(v_raw, kv_dtype)"),
    "q_scale_dropped": ('return decode_elements(w["q"], w["q_dtype"]) * float(w.get("q_scale", 1.0))',
                        'return decode_elements(w["q"], w["q_dtype"])'),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "attention.py")).read()
    assert src.count(old) == 1, (name, old)
    src = src.replace(old, new)
    mod = types.ModuleType(f"oracle._mutant_{name}")
    mod.__package__ = "oracle"
    mod.__file__ = os.path.join(ROOT, "oracle", f"_mutant_{name}.py")
    exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    return mod


def _pins_with_defaults(M):
    """Pins plus one that exercises default_sm_scale through batch_decode."""
    yield from PINS

    def pin_default_scale_brute(M):
        w = _tiny_decode(2)
        o, l = M.batch_decode(w)  # sm_scale defaulted inside
        ob, lb = brute_force(w, causal=False)  # 1/sqrt(d)
        np.testing.assert_allclose(o, ob, atol=1e-12)
    yield pin_default_scale_brute


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name):
    M = _mutant(name)
    failed = []
    for pin in _pins_with_defaults(M):
        try:
            pin(M)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
