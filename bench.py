"""Benchmark of the paged fp8-KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

A step is one fi_batch_decode_paged call (page-table gather, fp8 widening,
QK^T and PV on MFMA, online softmax, split-KV partials and their merge) on the
batch-decode workload: 64 requests, kv_len uniform in [512, 4096], 32 q / 8 kv
heads, head_dim 128, page 16 with shuffled pages, bf16 q/o, fp8 e4m3 K/V.
Inputs are resident in HBM before timing; the K/V pools are rotated over
several identical copies so that no step finds the previous step's pages in the
256 MB last-level cache.  The timed steps are captured once as a HIP graph and
replayed (a serving loop replays its captured decode step, so the host's launch
cost per call is outside the timed region); the per-call HIP events of an eager
run of the same steps give the roofline figure.
`value` is HBM GB/s counting the algorithmic bytes:
every valid K and V element once at 1 byte (fp8), q, o, lse and the page table
("fp8 KV cache in the in-tree prefill kernel", AMD-Ecosystem/flashinfer PR
#368, Tests, docs, benchmark: the fp8 byte count).

The same JSON line carries the causal-prefill figure (16 requests, qo_len
256..1024 plus a prefix of 0..2048, 32/8 heads, head_dim 128, e4m3 K/V, f16):
MFMA TFLOP/s at 4 * head_dim flops per visible (query, key) pair per q head,
and the same workload with its K/V stored contiguously per request through
the ragged call; beside them the long-context split-KV decode (8 requests of 32k..128k tokens,
64/8 heads, page 64, e5m2) and the batch-decode shapes with f16 q/o over f16,
bf16 (mixed 2-byte) and e4m3 caches, the batch-decode workload over e4m3fnuz and
e5m2fnuz caches, a plain device copy's bandwidth for
context, and the float64 oracle timed on the host cores on a bounded sample.
Roofline figures use the median of the per-call HIP events.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS_16 = 2500.0   # MI355X dense fp16 / bf16 MFMA
METRIC = "decode fp8-KV HBM GB/s (% of peak); prefill TFLOP/s (% of MFMA peak)"
ELEM = {"f16": 2, "bf16": 2, "e4m3": 1, "e5m2": 1, "e4m3fnuz": 1, "e5m2fnuz": 1}


def decode_bytes(w: dict) -> int:
    """Algorithmic bytes of one decode call."""
    eb = ELEM[w["kv_dtype"]]
    kv = int(w["kv_lens"].sum()) * w["num_kv_heads"] * w["head_dim"] * eb * 2
    ntok = int(w["qo_indptr"][-1])
    qo = ntok * w["num_qo_heads"] * w["head_dim"] * (ELEM[w["q_dtype"]] + ELEM[w["o_dtype"]])
    lse = ntok * w["num_qo_heads"] * 4
    table = 4 * (len(w["indices"]) + 2 * len(w["kv_lens"]) + 1)
    return kv + qo + lse + table


def visible_pairs(w: dict, causal: bool = True) -> int:
    tot = 0
    for qo, kv in zip(w["qo_lens"], w["kv_lens"]):
        qo, kv = int(qo), int(kv)
        if not causal:
            tot += qo * kv
            continue
        r = np.arange(qo)
        tot += int(np.clip(r + 1 + (kv - qo), 0, kv).sum())
    return tot


def prefill_flops(w: dict, causal: bool = True) -> int:
    return 4 * w["head_dim"] * w["num_qo_heads"] * visible_pairs(w, causal)


def _upload(w, dev, copies: int):
    import torch

    from attention_paged_fp8_amd import fi

    t2 = {"f16": torch.float16, "bf16": torch.bfloat16}

    def pool(x):
        t = torch.from_numpy(np.ascontiguousarray(x))
        if w["kv_dtype"] in t2:
            t = t.view(torch.int16).view(t2[w["kv_dtype"]])
        return t.to(dev)

    if w["q_dtype"] in t2:
        q = torch.from_numpy(w["q"].view(np.int16)).view(t2[w["q_dtype"]]).to(dev)
    else:  # fp8 query codes
        q = torch.from_numpy(np.ascontiguousarray(w["q"])).to(dev)
    idx = {n: torch.from_numpy(np.ascontiguousarray(w[n], dtype=np.int32)).to(dev)
           for n in ("indptr", "indices", "last_page_len", "qo_indptr")}
    kvs, keep = [], []
    for _ in range(copies):
        k, v = pool(w["k_pool"]), pool(w["v_pool"])
        s, kk = fi.make_paged_kv(k, v, idx["indptr"], idx["indices"], idx["last_page_len"], k_scale=w["k_scale"],
                                 v_scale=w["v_scale"], kv_dtype=w["kv_dtype"], indptr_h=w["indptr"],
                                 last_page_len_h=w["last_page_len"])
        kvs.append(s)
        keep.append((k, v, kk))
    return q, idx, kvs, keep


SETTLE_S = 0.5


def _settle(fn, n_copies, seconds=SETTLE_S):
    """Untimed calls until `seconds` of sustained load have passed.  The
    engine clock ramps up under load: right after the idle upload phase the
    compute-bound causal prefill takes ~20% longer (311-321 against 252 us,
    measured on MI355X), while the HBM-bound decode moves by ~1%; a serving
    loop runs at the sustained clock."""
    import torch

    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn(i % n_copies)
            i += 1
        torch.cuda.synchronize()
    return i


def _time_calls(fn, n_copies, steps, warmup, stream, settle=True):
    """Settle the clock under load (unless `settle` is false), warm up, then
    time exactly `steps` calls: wall clock bracketed by synchronize, and HIP
    events around every call on the launch stream."""
    import torch

    if settle:
        _settle(fn, n_copies)
    for i in range(warmup):
        fn(i % n_copies)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn(i % n_copies)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    return wall_ms, ev


def _graph_calls(fn, n_copies, steps, warmup):
    """The same `steps` calls captured into one HIP graph on a side stream
    (default priority) and replayed: wall clock of one replay bracketed by
    synchronize, per call -- the host's launch cost leaves the timed region, as
    in a serving loop that replays a captured decode step."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(warmup):
            fn(i % n_copies, side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
        for i in range(steps):
            fn(i % n_copies, side)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:  # the clock settles under the replayed load
        g.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    del g
    return wall_ms


def run_decode_bench(steps, warmup, copies, workload="batch_decode", kvd=None, graph=False):
    import torch

    from attention_paged_fp8_amd import fi
    from workloads import make_workload

    dev = torch.device("cuda:0")
    w = make_workload(workload, kvd=kvd)
    q, idx, kvs, keep = _upload(w, dev, copies)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    nws = fi.fi_decode_workspace_bytes(len(w["kv_lens"]), w["num_qo_heads"], w["head_dim"], int(w["kv_lens"].max()))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, st=stream):
        fi.fi_batch_decode_paged(q, kvs[i], o, lse=lse, workspace=ws, stream=st)

    wall_ms, ev = _time_calls(step, copies, steps, warmup, stream)
    if graph:
        try:
            return w, wall_ms, ev, _graph_calls(step, copies, steps, warmup)
        except Exception as e:  # no graph capture here: the eager wall clock stands in (reported as such)
            print(f"# graph capture failed ({type(e).__name__}: {e}); timing eager calls", file=sys.stderr, flush=True)
            torch.cuda.synchronize()
            return w, wall_ms, ev, None
    return w, wall_ms, ev


def run_prefill_bench(steps, warmup, ragged=False, fp8q=False, pv_fp8=False, copies=3, cold=False):
    """The causal prefill workload through the paged call, or (ragged) the
    same K/V values stored contiguously per request through the ragged call,
    or (fp8q) with its query quantised to e4m3 through the fp8-query call
    (pv_fp8: P V on the fp8 MFMA as well).  One call reads about 220 MB (q,
    K/V, o), less than the 256 MB last-level cache, so `copies` full sets of
    q, K/V, o and lse are rotated across the steps and no step finds the
    previous step's lines in that cache."""
    import torch

    from attention_paged_fp8_amd import fi
    from workloads import make_workload, ragged_rows

    dev = torch.device("cuda:0")
    w = make_workload("causal_prefill", q="e4m3" if fp8q else None)
    stream = torch.cuda.current_stream(dev)
    sets = []
    for _ in range(copies):
        q, idx, kvs, keep = _upload(w, dev, 0 if ragged else 1)
        o = torch.empty(q.shape, dtype=torch.float16, device=dev)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        kv = kvs[0] if kvs else None
        if ragged:
            kr, vr, indptr = ragged_rows(w)
            k, v = torch.from_numpy(kr).to(dev), torch.from_numpy(vr).to(dev)
            ind = torch.from_numpy(indptr).to(dev)
            kv, rkeep = fi.make_ragged_kv(k, v, ind, k_scale=w["k_scale"], v_scale=w["v_scale"],
                                          kv_dtype=w["kv_dtype"], indptr_h=indptr)
            keep = (keep, k, v, ind, rkeep)
        sets.append((q, idx, kv, o, lse, keep))

    def step(i):
        q, idx, kv, o, lse, _ = sets[i % copies]
        if fp8q:
            fi.fi_batch_prefill_paged_fp8q(q, idx["qo_indptr"], kv, o, q_dtype="e4m3", q_scale=w["q_scale"],
                                           o_dtype=w["o_dtype"], causal=True, pv_fp8=pv_fp8, lse=lse,
                                           qo_indptr_h=w["qo_indptr"], stream=stream)
        elif ragged:
            fi.fi_batch_prefill_ragged(q, idx["qo_indptr"], kv, o, causal=True, lse=lse,
                                       qo_indptr_h=w["qo_indptr"], stream=stream)
        else:
            fi.fi_batch_prefill_paged(q, idx["qo_indptr"], kv, o, causal=True, lse=lse,
                                      qo_indptr_h=w["qo_indptr"], stream=stream)

    cold_ev = None
    if cold:  # right after the upload, before the clock has settled: for comparison
        _, cold_ev = _time_calls(step, copies, steps, warmup, stream, settle=False)
    wall_ms, ev = _time_calls(step, copies, steps, warmup, stream)
    del sets
    torch.cuda.empty_cache()
    if cold:
        return w, wall_ms, ev, cold_ev
    return w, wall_ms, ev


def kernel_source_hash(kind: str) -> str:
    """sha256 over the sources that define a kernel (its .hip file, its body
    header and the shared device and internal headers)."""
    csrc = os.path.join(ROOT, "attention_paged_fp8_amd", "csrc")
    h = hashlib.sha256()
    for name in (f"fi_{kind}.hip", f"fi_{kind}_body.hpp", "fi_device.hpp", "fi_internal.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kind: str, workload: str):
    """HBM bytes per call from the committed counter summary
    profiles/<kind>_kernel.<workload>.traffic.txt (FETCH_SIZE and WRITE_SIZE
    per dispatch, each scaled by the reading of a plain copy of known size), or
    None when the summary is missing or was taken on other kernel sources."""
    path = os.path.join(PROFILES, f"{kind}_kernel.{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash(kind):
        return None
    try:
        return int(float(vals["hbm_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def copy_bandwidth(mb: int = 512, steps: int = 20) -> float:
    """GB/s of a plain device-to-device copy of `mb` MiB (read + write bytes):
    the practical streaming rate of this part, for context."""
    import torch

    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    _, ev = _time_calls(lambda i: dst.copy_(src), 1, steps, 3, stream)
    return 2 * n / (float(np.median(ev)) * 1e-3) / 1e9


def decode_extra(steps, warmup):
    """The single-decode workload (one request of 64 tokens: launch-bound, so
    its rate carries no roofline claim), long-context split-KV decode, the
    three KV types of the mixed-dtype decode workload, and the batch-decode
    workload over e4m3fnuz and e5m2fnuz caches: HIP-event medians and HBM rates
    (context beside the main line; each is a separate decode workload)."""
    out = {}
    for key, wl, kvd, copies in (("single_decode", "single_decode", None, 1),
                                 ("long_context", "long_context_decode", None, 2), ("kv_f16", "dtype_decode", "f16", 2),
                                 ("kv_bf16_mixed", "dtype_decode", "bf16", 2), ("kv_e4m3", "dtype_decode", "e4m3", 4),
                                 ("kv_e4m3fnuz", "batch_decode", "e4m3fnuz", 4),
                                 ("kv_e5m2fnuz", "batch_decode", "e5m2fnuz", 4)):
        w, wall_ms, ev = run_decode_bench(steps, warmup, copies, workload=wl, kvd=kvd)
        nb = decode_bytes(w)
        med = float(np.median(ev))
        out[key] = {"workload": w["name"] + (f"_kv_{kvd}" if kvd else ""), "bytes_per_call": nb,
                    "us_median": round(med * 1e3, 2), "gbs": round(nb / (med * 1e-3) / 1e9, 1),
                    "frac": None if key == "single_decode" else round(nb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"# {key}: {nb / 1e6:.1f} MB, median {med * 1e3:.1f} us -> {out[key]['gbs']} GB/s", file=sys.stderr,
              flush=True)
        import torch
        torch.cuda.empty_cache()
    return out


def run_pod_bench(steps, warmup, copies=3):
    """The mixed batch -- the causal-prefill workload (16 requests) and the
    batch-decode shapes with an f16 query over e4m3 (64 requests) -- three
    ways: one fi_batch_pod_paged call; the two separate calls back to back on
    one stream; the two calls on two streams of default priority, joined.
    HIP events on the launch stream around each whole step, after the clock
    has settled under load; `copies` full input sets rotated.  Returns medians
    in microseconds."""
    import torch

    from attention_paged_fp8_amd import fi
    from workloads import make_workload

    dev = torch.device("cuda:0")
    wp = make_workload("causal_prefill")
    wd = make_workload("dtype_decode", kvd="e4m3")
    main = torch.cuda.current_stream(dev)
    sp, sd = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    nws = fi.fi_decode_workspace_bytes(len(wd["kv_lens"]), wd["num_qo_heads"], wd["head_dim"], int(wd["kv_lens"].max()))
    sets = []
    for _ in range(copies):
        qp, ip, kvp, kp = _upload(wp, dev, 1)
        qd, idd, kvd, kd = _upload(wd, dev, 1)
        op = torch.empty(qp.shape, dtype=torch.float16, device=dev)
        lp = torch.empty(qp.shape[:2], dtype=torch.float32, device=dev)
        od = torch.empty(qd.shape, dtype=torch.float16, device=dev)
        ld = torch.empty(qd.shape[:2], dtype=torch.float32, device=dev)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        # the PagedKV structs point at both page tables (ip, idd): keep them with the set
        sets.append((qp, ip, kvp[0], op, lp, qd, kvd[0], od, ld, ws, kp, kd, idd))

    def pod(i):
        qp, ip, kvp, op, lp, qd, kvd, od, ld, ws = sets[i % copies][:10]
        fi.fi_batch_pod_paged(qp, ip["qo_indptr"], kvp, op, qd, kvd, od, causal=True, lse_p=lp, lse_d=ld,
                              qo_indptr_h=wp["qo_indptr"], workspace=ws, stream=main)

    def serial(i, st_p=None, st_d=None):
        qp, ip, kvp, op, lp, qd, kvd, od, ld, ws = sets[i % copies][:10]
        fi.fi_batch_prefill_paged(qp, ip["qo_indptr"], kvp, op, causal=True, lse=lp, qo_indptr_h=wp["qo_indptr"],
                                  stream=st_p or main)
        fi.fi_batch_decode_paged(qd, kvd, od, lse=ld, workspace=ws, stream=st_d or main)

    def two_streams(i):
        sp.wait_stream(main)
        sd.wait_stream(main)
        serial(i, sp, sd)
        main.wait_stream(sp)
        main.wait_stream(sd)

    out = {}
    for name, fn in (("pod_one_launch", pod), ("two_calls_one_stream", serial), ("two_calls_two_streams", two_streams)):
        _, ev = _time_calls(fn, copies, steps, warmup, main)
        out[name] = round(float(np.median(ev)) * 1e3, 2)
    torch.cuda.synchronize()
    del sets
    torch.cuda.empty_cache()
    return out


def run_copy_calibration(mb: int, reps: int = 5):
    """A plain device-to-device copy of `mb` MiB, `reps` times: the reference
    the FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    import torch

    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"# copy calibration: {reps} copies of {n} bytes", flush=True)


def host_info() -> dict:
    """The host's CPU model, core counts and the BLAS numpy runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(avail, share) if share > 0 else avail
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info

        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    if blas == "unknown":
        try:
            cfg = np.show_config(mode="dicts")
            b = cfg["Build Dependencies"]["blas"]
            blas = f"{b.get('name')} {b.get('version')}"
        except Exception:
            pass
    return dict(cpu_model=model, nproc=os.cpu_count(), cpus_available=avail, threads=threads, blas=blas)


def cpu_baseline(wd, runs: int = 3, prefill_requests=tuple(range(16))):
    """The float64 oracle on the host's cores (BLAS threads = the CPU share
    this process has: OMP_NUM_THREADS when set, else every available core),
    median of `runs` runs of each sample: the whole batch-decode workload
    (oracle GB/s over the same algorithmic bytes as the GPU figure) and
    requests `prefill_requests` of the causal-prefill workload (oracle
    GFLOP/s over their visible pairs)."""
    from threadpoolctl import threadpool_limits

    import oracle.attention as OA
    from workloads import make_workload

    info = host_info()
    nb = decode_bytes(wd)
    wp = make_workload("causal_prefill")
    sub = list(prefill_requests)
    qo, kv = wp["qo_lens"][sub], wp["kv_lens"][sub]
    pflops = prefill_flops(dict(wp, qo_lens=qo, kv_lens=kv))
    dt, pt = [], []
    with threadpool_limits(limits=info["threads"]):
        for _ in range(runs):
            t0 = time.perf_counter()
            OA.batch_decode(wd)
            dt.append(time.perf_counter() - t0)
            t0 = time.perf_counter()
            OA.batch_prefill(wp, causal=True, requests=sub)
            pt.append(time.perf_counter() - t0)
    d_s, p_s = float(np.median(dt)), float(np.median(pt))
    return dict(value=round(nb / d_s / 1e9, 4), unit="GB/s", cores=info["threads"], kind="oracle",
                sample=f"the whole batch-decode workload ({len(wd['kv_lens'])} requests, {nb / 1e6:.1f} MB "
                       f"algorithmic), float64 numpy, median of {runs} runs",
                seconds=[round(x, 3) for x in dt], nproc=info["nproc"], cpus_available=info["cpus_available"],
                cpu_model=info["cpu_model"], blas=info["blas"],
                prefill={"value": round(pflops / p_s / 1e9, 3), "unit": "GFLOP/s",
                         "sample": f"requests {sub} of the causal-prefill workload ({pflops / 1e9:.1f} GFLOP of "
                                   f"visible pairs), median of {runs} runs",
                         "seconds": [round(x, 3) for x in pt]})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=4, help="identical K/V pool copies rotated across steps")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-runs", type=int, default=3, help="runs of each oracle sample (median reported)")
    ap.add_argument("--only", choices=("all", "decode", "prefill", "pod"), default="all",
                    help="run one path only (for per-kernel counter passes)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the long-context and mixed-dtype decode workloads and the copy bandwidth")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: this library and benchmark run on one GPU only; "
              "multi-GPU sharding is not implemented", file=sys.stderr)
        sys.exit(2)

    if args.calib_copy:
        run_copy_calibration(args.calib_copy)
        return

    from attention_paged_fp8_amd import fi

    if not os.path.exists(fi.LIB_PATH):
        from attention_paged_fp8_amd.build import build
        build()

    from workloads import make_workload

    w, eager_ms, ev, graph_ms = make_workload("batch_decode"), float("nan"), np.array([float("nan")]), float("nan")
    if args.only in ("all", "decode"):
        w, eager_ms, ev, graph_ms = run_decode_bench(args.steps, args.warmup, args.copies, graph=True)
    elif args.only == "pod":
        graph_ms = None
    nbytes = decode_bytes(w)
    # whole-job rate: the timed steps replayed as one captured graph (eager calls if capture failed)
    graphed = graph_ms is not None
    wall_ms = graph_ms if graphed else eager_ms
    value = nbytes / (wall_ms * 1e-3) / 1e9
    ev_ms = float(np.median(ev))
    achieved = nbytes / (ev_ms * 1e-3) / 1e9
    print(f"# decode: {nbytes / 1e6:.1f} MB per call, graph replay {wall_ms * 1e3 if graphed else float('nan'):.1f} us/step, eager calls "
          f"{eager_ms * 1e3:.1f} us/step, events median {ev_ms * 1e3:.1f} us (mean {ev.mean() * 1e3:.1f}, "
          f"min {ev.min() * 1e3:.1f}, max {ev.max() * 1e3:.1f})", file=sys.stderr, flush=True)

    prefill = None
    if args.only in ("all", "prefill"):
        pw, p_wall, p_ev, p_cold = run_prefill_bench(args.prefill_steps, 3, cold=True)
        flops = prefill_flops(pw)
        p_ms = float(np.median(p_ev))
        c_ms = float(np.median(p_cold))
        tflops = flops / (p_ms * 1e-3) / 1e12
        print(f"# prefill: {flops / 1e9:.1f} GFLOP per call, events median {p_ms * 1e3:.1f} us -> {tflops:.1f} TFLOP/s "
              f"(before the clock settles: {c_ms * 1e3:.1f} us)", file=sys.stderr, flush=True)
        prefill = {
            "workload": pw["name"], "tflops": round(tflops, 2), "ms": round(p_ms, 5),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS_16,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS_16, 4),
                         "traffic": measured_traffic("prefill", pw["name"]), "flops_per_launch": flops},
            "dtype": "f16",
            "cold_ms": round(c_ms, 5),
            "cold_tflops": round(flops / (c_ms * 1e-3) / 1e12, 2),
            "cold_note": "the same calls timed right after the upload with only the warm-up steps, before the engine "
                         "clock has settled under load",
            "copies_rotated": 3,
            "rotation": "3 full sets of q, K/V pools, o and lse (about 220 MB each) rotated across the steps, so no "
                        "step finds the previous step's lines in the 256 MB last-level cache",
        }
        if not args.no_extra:
            _, _, r_ev = run_prefill_bench(args.prefill_steps, 3, ragged=True)
            r_ms = float(np.median(r_ev))
            prefill["ragged"] = {"ms": round(r_ms, 5), "tflops": round(flops / (r_ms * 1e-3) / 1e12, 2)}
            print(f"# prefill, ragged K/V: events median {r_ms * 1e3:.1f} us", file=sys.stderr, flush=True)
            _, _, f_ev = run_prefill_bench(args.prefill_steps, 3, fp8q=True)
            f_ms = float(np.median(f_ev))
            prefill["fp8_query"] = {"ms": round(f_ms, 5), "tflops": round(flops / (f_ms * 1e-3) / 1e12, 2),
                                    "note": "QK on the fp8 MFMA, PV in f16"}
            print(f"# prefill, fp8 query: events median {f_ms * 1e3:.1f} us -> {flops / (f_ms * 1e-3) / 1e12:.1f} "
                  "TFLOP/s", file=sys.stderr, flush=True)
            _, _, g_ev = run_prefill_bench(args.prefill_steps, 3, fp8q=True, pv_fp8=True)
            g_ms = float(np.median(g_ev))
            prefill["fp8_query_fp8_pv"] = {"ms": round(g_ms, 5), "tflops": round(flops / (g_ms * 1e-3) / 1e12, 2),
                                           "note": "QK and PV on the fp8 MFMA, P rounded to e4m3"}
            print(f"# prefill, fp8 query and fp8 P V: events median {g_ms * 1e3:.1f} us -> "
                  f"{flops / (g_ms * 1e-3) / 1e12:.1f} TFLOP/s", file=sys.stderr, flush=True)

    extra, copy_gbs, pod = None, None, None
    if args.only in ("all", "pod") and not args.no_extra:
        pod = run_pod_bench(args.prefill_steps, 3)
        pod["workload"] = ("causal_prefill_b16_qo256-1024_prefix0-2048_h32-8_d128_page16_e4m3_f16 + "
                           "dtype_decode_b64_kv512-4096_h32-8_d128_page16_f16q_kv_e4m3")
        pod["unit"] = "us (median of HIP events around the whole step)"
        print(f"# mixed prefill + decode batch: one POD launch {pod['pod_one_launch']} us, two calls on one stream "
              f"{pod['two_calls_one_stream']} us, on two streams {pod['two_calls_two_streams']} us", file=sys.stderr,
              flush=True)
    if args.only == "all" and not args.no_extra:
        extra = decode_extra(args.steps, 3)
        copy_gbs = round(copy_bandwidth(), 1)
        print(f"# plain device copy: {copy_gbs} GB/s", file=sys.stderr, flush=True)

    cpu = None if (args.no_cpu or args.only in ("prefill", "pod")) else cpu_baseline(w, args.cpu_runs)
    if cpu is not None and prefill is not None:
        prefill["cpu_baseline"] = cpu["prefill"]
    if cpu is not None:
        print(f"# oracle on {cpu['cores']} threads ({cpu['cpu_model']}, {cpu['blas']}): decode {cpu['value']} GB/s, "
              f"prefill {cpu['prefill']['value']} GFLOP/s", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC,
        "value": round(value, 2) if np.isfinite(value) else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5) if np.isfinite(wall_ms) else None,
        "timing": (("the timed steps captured as one HIP graph and replayed" if graphed else
                    "the timed steps as eager calls (graph capture failed)") +
                   ", wall clock bracketed by synchronize; roofline from the median of per-call HIP events in an "
                   f"eager run; every leg first runs {SETTLE_S} s of untimed calls so the engine clock settles under "
                   "load, then the warm-up steps"),
        "eager_ms_per_step": round(eager_ms, 5) if np.isfinite(eager_ms) else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w["name"], "batch": 64, "kv_len": "uniform[512,4096]", "total_kv_tokens": int(w["kv_lens"].sum()),
            "num_qo_heads": 32, "num_kv_heads": 8, "head_dim": 128, "page_size": 16, "pages": "shuffled",
            "q_o": "bf16", "kv": "fp8 e4m3 (OCP)", "seed": 2, "kv_pool_copies_rotated": args.copies,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode", w["name"]),
            "kernel": "decode_kernel + merge_kernel (one C-ABI call; median of HIP events on its stream)",
            "bytes_per_launch": nbytes,
        },
        "prefill": prefill,
        "decode_other": extra,
        "pod": pod,
        "copy_gbs": copy_gbs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
