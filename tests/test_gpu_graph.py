"""Decode and prefill calls captured into a HIP graph and replayed.

A serving loop replays a captured decode (or prefill) step instead of paying
the host's launch cost per call.  Everything a call needs is planned on the
host and travels in the kernel arguments, so a captured call replays the same
work on whatever the buffers hold at replay time.  Each test captures the
calls once, then replays the graph several times with eager work between the
replays (a new query written into the captured buffer, an eager call on other
buffers, synchronizations) and checks every replay bitwise against an eager
call on the same inputs, and against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle.attention as OA
from attention_paged_fp8_amd import fi
from workloads import make_workload
from gpu_util import T2, assert_parity, paged_kv, say, upload, workspace_for

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _queries(w, n, device):
    """n seeded query tensors of the workload's shape and dtype (the first is
    the workload's own)."""
    rng = np.random.default_rng(1234)
    out = []
    for i in range(n):
        if i == 0:
            bits = w["q"]
        else:
            x = rng.standard_normal(w["q"].shape).astype(np.float32)
            bits = torch.from_numpy(x).to(T2[w["q_dtype"]]).view(torch.int16).numpy()
        out.append(torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(T2[w["q_dtype"]]).to(device))
    return out


def _capture(fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream, capture_error_mode="thread_local"):
        fn(stream)
    return g


@pytest.mark.parametrize("wl", ["batch_decode", "long_context_decode"])
def test_decode_graph_replays(gpu_device, wl):
    say("graph decode", wl)
    w = make_workload(wl)
    d = upload(w, gpu_device)
    kv, keep = paged_kv(w, d)
    B, H, D = len(w["kv_lens"]), w["num_qo_heads"], w["head_dim"]
    ws = workspace_for(w, gpu_device)
    q_in = torch.empty_like(d["q"])
    o = torch.empty((B, H, D), dtype=T2[w["o_dtype"]], device=gpu_device)
    lse = torch.empty((B, H), dtype=torch.float32, device=gpu_device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    q_in.copy_(d["q"])
    torch.cuda.synchronize()
    with torch.cuda.stream(side):  # warm the library's per-device caches outside the capture
        fi.fi_batch_decode_paged(q_in, kv, o, lse=lse, workspace=ws, stream=side)
    torch.cuda.synchronize()
    g = _capture(lambda st: fi.fi_batch_decode_paged(q_in, kv, o, lse=lse, workspace=ws, stream=st), side)
    torch.cuda.synchronize()

    qs = _queries(w, REPLAYS, gpu_device)
    ws_e = workspace_for(w, gpu_device)
    for r in range(REPLAYS):
        q_in.copy_(qs[r])  # eager work between replays
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e = torch.full_like(o, float("nan"))
        l_e = torch.full_like(lse, float("nan"))
        fi.fi_batch_decode_paged(qs[r], kv, o_e, lse=l_e, workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_e.view(torch.int16)), f"replay {r}: output differs from eager"
        assert torch.equal(lse, l_e), f"replay {r}: lse differs from eager"
        if r == 0 and wl == "batch_decode":  # the long-context workload's full oracle is covered by the decode tests
            o_ref, l_ref = OA.batch_decode(w)
            assert_parity(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, l_ref, w["o_dtype"],
                          f"graph replay, {wl}")
    del g


def test_prefill_graph_replays(gpu_device):
    say("graph prefill causal-prefill workload")
    w = make_workload("causal_prefill")
    d = upload(w, gpu_device)
    kv, keep = paged_kv(w, d)
    T, H, D = int(w["qo_indptr"][-1]), w["num_qo_heads"], w["head_dim"]
    q_in = torch.empty_like(d["q"])
    o = torch.empty((T, H, D), dtype=T2[w["o_dtype"]], device=gpu_device)
    lse = torch.empty((T, H), dtype=torch.float32, device=gpu_device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    q_in.copy_(d["q"])
    torch.cuda.synchronize()

    def call(st, q=q_in, out=o, l=lse):
        fi.fi_batch_prefill_paged(q, d["qo_indptr"], kv, out, causal=True, lse=l, qo_indptr_h=w["qo_indptr"],
                                  stream=st)

    with torch.cuda.stream(side):
        call(side)
    torch.cuda.synchronize()
    g = _capture(call, side)
    torch.cuda.synchronize()

    qs = _queries(w, REPLAYS, gpu_device)
    for r in range(REPLAYS):
        q_in.copy_(qs[r])
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e = torch.full_like(o, float("nan"))
        l_e = torch.full_like(lse, float("nan"))
        call(torch.cuda.current_stream(), q=qs[r], out=o_e, l=l_e)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_e.view(torch.int16)), f"replay {r}: output differs from eager"
        assert torch.equal(lse, l_e), f"replay {r}: lse differs from eager"
        if r == 0:
            rng = np.random.default_rng(7)  # sampled (token, head) outputs of the oracle, one by one
            toks = rng.integers(0, T, 64)
            heads = rng.integers(0, H, 64)
            o_s, l_s = OA.attention_rows(w, toks, heads, causal=True)
            o_np, l_np = o.double().cpu().numpy(), lse.double().cpu().numpy()
            assert_parity(o_np[toks, heads], l_np[toks, heads], o_s, l_s, w["o_dtype"], "graph replay, prefill rows")
    del g


def _replay_against_eager(capture_call, eager_call, q_in, queries, outs):
    """Capture capture_call(stream) once; for each query tensor write it into
    q_in eagerly, replay, and compare every output bitwise with
    eager_call(query) on fresh buffers.  Returns the first replay's outputs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    q_in.copy_(queries[0])
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        capture_call(side)
    torch.cuda.synchronize()
    g = _capture(capture_call, side)
    torch.cuda.synchronize()
    first = None
    for r, qr in enumerate(queries):
        q_in.copy_(qr)
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager_call(qr)
        torch.cuda.synchronize()
        for t, e in zip(outs, ref):
            assert torch.equal(t.view(torch.int16) if t.element_size() == 2 else t,
                               e.view(torch.int16) if e.element_size() == 2 else e), f"replay {r} differs from eager"
        if first is None:
            first = [t.clone() for t in outs]
    del g
    return first


@pytest.mark.parametrize("variant", ["fp8q", "fp8q_pv8", "ragged"])
def test_prefill_variant_graph_replays(gpu_device, variant):
    """The fp8-query prefill (P V in f16, and on the fp8 MFMA) and the ragged
    prefill, captured and replayed like the paged call."""
    say("graph prefill", variant)
    from workloads import make_paged, ragged_rows
    q = "e4m3" if variant.startswith("fp8q") else "f16"
    w = make_paged(31, qo_lens=[1, 70, 300, 129], prefix_lens=[0, 45, 600, 3], hq=32, hkv=8, d=128, page=16,
                   q=q, kvd="e4m3", o="f16" if q == "e4m3" else None)
    d = upload(w, gpu_device)
    T, H, D = int(w["qo_indptr"][-1]), w["num_qo_heads"], w["head_dim"]
    q_in = torch.empty_like(d["q"])
    o = torch.empty((T, H, D), dtype=torch.float16, device=gpu_device)
    lse = torch.empty((T, H), dtype=torch.float32, device=gpu_device)
    if variant == "ragged":
        kr, vr, indptr = ragged_rows(w)
        kt, vt = torch.from_numpy(kr).to(gpu_device), torch.from_numpy(vr).to(gpu_device)
        ind = torch.from_numpy(indptr).to(gpu_device)
        kv, keep = fi.make_ragged_kv(kt, vt, ind, k_scale=w["k_scale"], v_scale=w["v_scale"], kv_dtype="e4m3",
                                     indptr_h=indptr)
    else:
        kv, keep = paged_kv(w, d)

    def call(qq, out, l, st=None):
        if variant == "ragged":
            fi.fi_batch_prefill_ragged(qq, d["qo_indptr"], kv, out, causal=True, lse=l, qo_indptr_h=w["qo_indptr"],
                                       stream=st)
        else:
            fi.fi_batch_prefill_paged_fp8q(qq, d["qo_indptr"], kv, out, q_dtype=q, q_scale=w["q_scale"], causal=True,
                                           pv_fp8=variant == "fp8q_pv8", lse=l, qo_indptr_h=w["qo_indptr"], stream=st)

    def eager(qq):
        oe, le = torch.full_like(o, float("nan")), torch.full_like(lse, float("nan"))
        call(qq, oe, le)
        return oe, le

    if q == "e4m3":  # further queries: the same codes with the rows permuted
        perm = np.random.default_rng(9).permutation(T)
        queries = [d["q"], d["q"][torch.from_numpy(perm).to(gpu_device)].contiguous()]
    else:
        queries = _queries(w, 2, gpu_device)
    first = _replay_against_eager(lambda st: call(q_in, o, lse, st), eager, q_in, queries, [o, lse])
    if variant != "fp8q_pv8":  # the fp8 P V tolerance is covered by the fp8-query tests
        o_ref, l_ref = OA.batch_prefill(w, causal=True)
        assert_parity(first[0].double().cpu().numpy(), first[1].double().cpu().numpy(), o_ref, l_ref, "f16",
                      f"graph replay, {variant}")


def test_fnuz_decode_graph_replays(gpu_device):
    """e4m3fnuz decode (fast and exact widening chosen per wave and step at
    run time) captured and replayed."""
    say("graph decode e4m3fnuz")
    from workloads import make_paged
    w = make_paged(33, kv_lens=[1500, 33, 900, 2048, 7, 640], hq=32, hkv=8, d=128, page=16, q="bf16", kvd="e4m3fnuz")
    d = upload(w, gpu_device)
    kv, keep = paged_kv(w, d)
    B, H, D = len(w["kv_lens"]), w["num_qo_heads"], w["head_dim"]
    ws = workspace_for(w, gpu_device)
    q_in = torch.empty_like(d["q"])
    o = torch.empty((B, H, D), dtype=torch.bfloat16, device=gpu_device)
    lse = torch.empty((B, H), dtype=torch.float32, device=gpu_device)
    ws_e = workspace_for(w, gpu_device)

    def eager(qq):
        oe, le = torch.full_like(o, float("nan")), torch.full_like(lse, float("nan"))
        fi.fi_batch_decode_paged(qq, kv, oe, lse=le, workspace=ws_e)
        return oe, le

    first = _replay_against_eager(lambda st: fi.fi_batch_decode_paged(q_in, kv, o, lse=lse, workspace=ws, stream=st),
                                  eager, q_in, _queries(w, REPLAYS, gpu_device), [o, lse])
    o_ref, l_ref = OA.batch_decode(w)
    assert_parity(first[0].double().cpu().numpy(), first[1].double().cpu().numpy(), o_ref, l_ref, "bf16",
                  "graph replay, e4m3fnuz decode")
