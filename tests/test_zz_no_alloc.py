"""GPU test of fi_batch_decode_paged_noalloc, the decode call that allocates
nothing and keeps its split-KV state in the library's per-device scratch
array: through the C ABI, two calls in a row (the second on a smaller batch),
each bit-identical to fi_batch_decode_paged with a caller's workspace on the
same inputs, and within the float64 oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from attention_paged_fp8_amd import fi
from workloads import make_paged
from gpu_util import T2, assert_parity, paged_kv, say, upload, workspace_for

pytestmark = pytest.mark.gpu


def _both(w, d):
    """(o, lse) of the allocation-free call and of the workspace call."""
    B, H, D = len(w["kv_lens"]), w["num_qo_heads"], w["head_dim"]
    kv, keep = paged_kv(w, d)
    out = []
    for noalloc in (True, False):
        o = torch.full((B, H, D), float("nan"), dtype=T2[w["o_dtype"]], device=d["q"].device)
        lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=d["q"].device)
        if noalloc:
            fi.fi_batch_decode_paged_noalloc(d["q"], kv, o, lse=lse)
        else:
            fi.fi_batch_decode_paged(d["q"], kv, o, lse=lse, workspace=workspace_for(w, d["q"].device))
        torch.cuda.synchronize()
        out.append((o.double().cpu().numpy(), lse.double().cpu().numpy()))
    return out


def test_noalloc_matches_workspace_call_twice(gpu_device):
    # first call: 48 requests of 512..4096 tokens, 32/8 heads, e4m3 (a balanced split with a merge)
    say("noalloc decode, call 1 (48 requests)")
    w1 = make_paged(61, kv_range=(512, 4096), batch=48, hq=32, hkv=8, d=128, page=16, q="bf16", kvd="e4m3")
    d1 = upload(w1, gpu_device)
    (o_a, l_a), (o_b, l_b) = _both(w1, d1)
    assert np.array_equal(o_a, o_b) and np.array_equal(l_a, l_b), "call 1 differs from the workspace call"
    o_ref, l_ref = OA.batch_decode(w1)
    assert_parity(o_a, l_a, o_ref, l_ref, "bf16", "noalloc call 1")
    # second call, smaller: 5 requests (one empty), 16/4 heads, head_dim 64, e5m2, page 32
    say("noalloc decode, call 2 (5 requests)")
    w2 = make_paged(62, kv_lens=[300, 0, 2000, 17, 900], hq=16, hkv=4, d=64, page=32, q="f16", kvd="e5m2")
    d2 = upload(w2, gpu_device)
    (o_a, l_a), (o_b, l_b) = _both(w2, d2)
    assert np.array_equal(o_a, o_b) and np.array_equal(l_a, l_b), "call 2 differs from the workspace call"
    o_ref, l_ref = OA.batch_decode(w2)
    assert_parity(o_a, l_a, o_ref, l_ref, "f16", "noalloc call 2")
    assert np.all(o_a[1] == 0) and np.all(np.isneginf(l_a[1]))
