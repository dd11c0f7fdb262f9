"""CPU checks of the seeded input generators' layout helpers (no GPU).

The ragged layout used by the ragged-K/V and single-request prefill tests must
hold exactly the stored elements of the paged workload it is built from, each
request's tokens contiguous and in logical order, with poison outside the
requests' rows.
"""
import numpy as np
import pytest

import oracle.attention as OA
from workloads import NAN_BITS, make_paged, ragged_rows


@pytest.mark.parametrize("kvd,page", [("e4m3", 16), ("f16", 4), ("e5m2", 1)])
def test_ragged_rows_match_paged_gather(kvd, page):
    w = make_paged(3, qo_lens=[4, 0, 9, 2], kv_lens=[37, 5, 0, 16], hq=4, hkv=2, d=8, page=page, q="f16", kvd=kvd,
                   extra_pages=3)
    k, v, indptr = ragged_rows(w, lead=3, tail=2)
    assert indptr.tolist() == [3, 40, 45, 45, 61]
    assert k.shape == (63, 2, 8) and v.shape == k.shape and k.dtype == w["k_pool"].dtype
    for i in range(4):
        for rows, pool in ((k, w["k_pool"]), (v, w["v_pool"])):
            ref = OA.gather_request(pool, w["indptr"], w["indices"], w["last_page_len"], page, i)
            assert np.array_equal(rows[indptr[i]:indptr[i + 1]], ref)
    poison = NAN_BITS[kvd]
    for rows in (k, v):
        assert np.all(rows[:3] == poison) and np.all(rows[61:] == poison)


def test_ragged_rows_give_the_paged_attention():
    """The oracle over the ragged rows equals the oracle over the pages."""
    w = make_paged(4, qo_lens=[5, 3], prefix_lens=[20, 0], hq=4, hkv=2, d=8, page=4, q="bf16", kvd="e4m3")
    k, v, indptr = ragged_rows(w, lead=1)
    o_ref, l_ref = OA.batch_prefill(w, causal=True)
    q = OA.decode_elements(w["q"], "bf16")
    for i in range(2):
        a, b = int(w["qo_indptr"][i]), int(w["qo_indptr"][i + 1])
        kr = OA.decode_elements(k[indptr[i]:indptr[i + 1]], "e4m3") * float(w["k_scale"])
        vr = OA.decode_elements(v[indptr[i]:indptr[i + 1]], "e4m3") * float(w["v_scale"])
        o, l = OA.attention(q[a:b], kr, vr, causal=True, sm_scale=OA.default_sm_scale(8))
        assert np.array_equal(o, o_ref[a:b]) and np.array_equal(l, l_ref[a:b])
