"""Benchmark of one GPU's share of the fused bf16 GEMM + reduce-scatter.

One step = one fused call (local GEMM, bf16 send chunks with ready flags,
owned-shard sum of the staged peer partials) over one batch of synthetic
inputs resident in HBM.  Ready words count calls, so nothing is cleared
between steps; after the run every ready word of a buffer set equals the
number of calls made on it.  Prints ONE JSON line.

Default workload: P = 8, rank 3, M = N = 4096, K = 512 (the HBM-bound,
communication-dominant case), rotating buffer sets so the 256 MB
last-level cache cannot serve the inputs.  The three M = N = 32768 shares
(K = 2048, 4096 and 8192) are measured in the same run and reported under
"secondary", each with at least 20 timed launches, its roofline and its own
CPU-oracle baseline on a stated row block; the K = 8192 share is first swept
over its 12 schedule points (chunk_rows x tile order) and reported at the
best one.

roofline.traffic is the fused kernel's measured HBM traffic per launch, read
from profiles/pmc_traffic.txt (rocprofv3 FETCH_SIZE and WRITE_SIZE, each
scaled by what the counter reads for a plain device copy of known size, see
--copy-calibration); it is null when that file was taken from other kernel
sources than the ones in the tree.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-secondary]
    python bench.py --copy-calibration     # 5 device copies of 512 MiB, for the counters
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused GEMM+RS TFLOP/s & epilogue GB/s per GPU; % of MFMA/HBM roofline"
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="comm_dominant")
    p.add_argument("--tile-order", type=int, default=None)
    p.add_argument("--chunk-rows", type=int, default=None)
    p.add_argument("--config", type=int, default=0)
    p.add_argument("--group-n", type=int, default=0)
    p.add_argument("--max-workgroups", type=int, default=0)
    p.add_argument("--owned-split", type=int, default=0, choices=(-1, 0, 1),
                   help="owned shard in 64x128 sub-tiles: 1 on, -1 off, 0 library default")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run 5 device copies of 512 MiB (counter calibration) and exit")
    p.add_argument("--write-traffic", default=None, metavar="DIR",
                   help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs found under DIR "
                        "(<workload>_fetch, <workload>_write, copy_fetch, copy_write) into "
                        "profiles/pmc_traffic.txt for the current kernel sources, and exit")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ag-gemm", action="store_true",
                   help="skip the all-gather + GEMM measurement (N x N/8 x N, N = 32768)")
    p.add_argument("--no-push", action="store_true",
                   help="skip the atomic push variant beside the staged share")
    p.add_argument("--no-consumer", action="store_true",
                   help="skip the chunk-consumer measurement beside the producer")
    p.add_argument("--no-gemm-only", action="store_true")
    p.add_argument("--store-policy", type=int, default=0, choices=(0, 1, 2),
                   help="output store cache policy: 0 auto, 1 streaming, 2 without the hint")
    p.add_argument("--no-reduce", action="store_true",
                   help="skip the inter-CU reduction role beside the staged share")
    p.add_argument("--sweep", action="store_true",
                   help="large-K schedule sweep: chunk_rows x tile order, one JSON line each")
    p.add_argument("--timeline", action="store_true",
                   help="phase times and CU placement of every workgroup, from the "
                        "instrumented timing build (libpk_gemm_rs_timeline.so); one JSON line")
    return p.parse_args()


class BufferSet:
    def __init__(self, w, seed, chunk_rows, torch, gen, pk):
        dev = "cuda"
        self.A, self.B, self.peers = gen.make_inputs(w, dev, seed=seed)
        self.send = torch.empty((w.P - 1, w.S, w.N), dtype=torch.bfloat16, device=dev)
        odt = torch.float32 if w.out_dtype == "f32" else torch.bfloat16
        self.out = torch.empty((w.S, w.N), dtype=odt, device=dev)
        self.flags = torch.zeros(pk.pk_flags_words(w.P, w.M, chunk_rows), dtype=torch.int32,
                                 device=dev)
        self.gemm_out = None

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in
                   (self.A, self.B, self.peers, self.send, self.out))


def time_steps(fn, n_sets, warmup, steps, torch):
    """Run warmup + timed steps; returns (ms per step, wall seconds).

    A step is one launch of the kernel, issued through a pre-bound call so the
    host stays ahead of the GPU; HIP events on the launch stream bracket the
    whole timed region, so ms per step is the kernel's average duration in a
    back-to-back stream of launches (inter-launch gaps included).
    """
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        fn((warmup + i) % n_sets)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return t_start.elapsed_time(t_end) / steps, wall


def ready_words(w, chunk_rows):
    """Ready words at the front of the flags buffer, one per chunk of each
    send slot; the counters after them are zero between calls."""
    return (w.P - 1) * (w.S // chunk_rows) if w.S > 0 else 0


def measure(w, args, torch, gen, pk, metrics, steps, warmup, rotate=True, gemm_only=True,
            tile_order=None, chunk_rows=None, reduce_counts=(), reduce_order=None):
    chunk = chunk_rows or args.chunk_rows or w.chunk_rows
    if tile_order is None:
        tile_order = args.tile_order
    order = w.tile_order if tile_order is None else tile_order
    set_bytes = w.algorithmic_bytes()
    n_sets = 1
    if rotate and set_bytes < 2 * MALL_BYTES:
        n_sets = max(2, min(8, math.ceil(1.2 * MALL_BYTES / set_bytes)))
    sets = [BufferSet(w, 17 * i, chunk, torch, gen, pk) for i in range(n_sets)]
    out_bf16 = 1 if w.out_dtype == "bf16" else 0
    opts = dict(config=args.config, max_workgroups=args.max_workgroups, group_n=args.group_n,
                store_policy=args.store_policy)
    fused_opts = dict(opts, owned_split=args.owned_split)

    calls = [0] * n_sets
    launch = [pk.BoundCall(s.A, s.B, s.peers, s.send, s.out, s.flags, w.M, w.N, w.K, w.P,
                           w.rank, chunk, order, out_bf16, **fused_opts) for s in sets]

    def step(i):
        launch[i]()
        calls[i] += 1

    ms_step, wall = time_steps(step, n_sets, warmup, steps, torch)
    k_ms = ms_step
    # every ready word counts the calls on its set; every counter is back to 0
    nr = ready_words(w, chunk)
    for s, n in zip(sets, calls):
        assert int(s.flags[:nr].min()) == n and int(s.flags[:nr].max()) == n
        assert int(s.flags[nr:].abs().max()) == 0
    res = dict(ms_per_step=ms_step, kernel_ms=k_ms, wall_s=wall, n_sets=n_sets,
               chunk_rows=chunk, tile_order=order)
    if gemm_only:
        for s in sets:
            s.gemm_out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")

        glaunch = [pk.BoundCall(s.A, s.B, None, None, s.gemm_out, None, w.M, w.N, w.K, w.P,
                                0, 0, 0, 1, gemm_only=True, **opts) for s in sets]
        g_ms, _ = time_steps(lambda i: glaunch[i](), n_sets, warmup, steps, torch)
        res["gemm_only_kernel_ms"] = g_ms
        res["exposed_fraction"] = metrics.exposed_fraction(k_ms, g_ms)
    if reduce_counts and w.P > 1:
        res["inter_cu_reduce"] = measure_reduce(w, sets, calls, chunk,
                                                order if reduce_order is None else reduce_order,
                                                out_bf16,
                                                fused_opts, reduce_counts, steps, warmup, k_ms,
                                                torch, pk)
    del sets
    torch.cuda.empty_cache()
    return res


def measure_reduce(w, sets, calls, chunk, order, out_bf16, opts, counts, steps, warmup,
                   fused_ms, torch, pk):
    """The inter-CU schedule's reduction role on the same buffer sets as the
    staged share: n workgroups sum the owned shard's peer partials into an
    fp32 workspace of its own while the rest compute; n = 0 sums them in the
    background of the main loops instead.  Timed back to back for each n
    like the share; the error words are checked after the timed steps."""
    n_sets = len(sets)
    words = pk.pk_reduce_piece_words(w.M, w.N, w.P)
    side = []
    for s in sets:
        presum = torch.empty((w.S, w.N), dtype=torch.float32, device="cuda")
        side.append((presum, torch.zeros(words, dtype=torch.int32, device="cuda"),
                     torch.zeros(1, dtype=torch.int32, device="cuda")))
    red_calls = [0] * n_sets
    res = {}
    for nc in counts:
        launch = [pk.BoundInterCUReduce(s.A, s.B, s.peers, s.send, s.out, s.flags, ps, pw, er,
                                        w.M, w.N, w.K, w.P, w.rank, chunk, order, out_bf16,
                                        red_calls[i] + 1, nc, **opts)
                  for i, (s, (ps, pw, er)) in enumerate(zip(sets, side))]

        def step(i):
            launch[i]()
            launch[i].next()
            red_calls[i] += 1
            calls[i] += 1
        ms, _ = time_steps(step, n_sets, warmup, steps, torch)
        for call in launch:
            assert call.check() == 0, "a reduction wait gave up"
        res[str(nc)] = round(ms * 1e3, 2) if ms < 1 else round(ms, 4)
    nw = ready_words(w, chunk)
    for s, (ps, pw, er), n, nr in zip(sets, side, calls, red_calls):
        assert int(s.flags[:nw].min()) == n and int(s.flags[nw:].abs().max()) == 0
        assert int(pw.min()) == nr and int(pw.max()) == nr and int(er.item()) == 0
    best = min(res, key=res.get)
    unit = "us_per_call_by_comm_cus" if fused_ms < 1 else "ms_per_call_by_comm_cus"
    scale = 1e3 if fused_ms < 1 else 1.0
    return {"tile_order": order, unit: res, "best_comm_cus": int(best),
            "vs_fused": round(res[best] / (fused_ms * scale), 3)}


def measure_push(w, args, torch, gen, pk, steps, warmup):
    """The atomic push variant on the same share: fp32 atomic adds of every
    tile into the owners' accumulators [P][S][N], timed like the staged
    share (back-to-back launches, events over the region)."""
    s = BufferSet(w, 17, w.chunk_rows, torch, gen, pk)
    accum = torch.zeros((w.P, w.S, w.N), dtype=torch.float32, device="cuda")
    call = pk.BoundPush(s.A, s.B, accum, s.flags, w.M, w.N, w.K, w.P, w.rank, w.chunk_rows,
                        w.tile_order)
    ms, _ = time_steps(lambda i: call(), 1, warmup, steps, torch)
    # bytes the adds move: every accumulator word read and written once
    rmw = 2 * 4 * w.M * w.N
    return {"kernel_ms": round(ms, 5), "accum_rmw_bytes": rmw,
            "accum_rmw_gbps": round(rmw / (ms * 1e-3) / 1e9, 1)}


def measure_ag_gemm(torch, gen, pk, steps, warmup, n=32768, P=8, rank=3, chunk_rows=512):
    """All-gather + GEMM at the pages' tensor-parallel shape (N x N/8 x N with
    N = 32768: C [N][N/8] = A_gathered [N][N] * B [N][N/8]), every chunk
    already arrived (ready words preset), so the time is the GEMM plus the
    per-tile waits; the GEMM-only mode on the same shape is timed beside it."""
    w = gen.Workload("ag_gemm", P=1, rank=0, M=n, N=n // 8, K=n, chunk_rows=0,
                     ab_dist="normal_sqrtk", peer_dist="normal", out_dtype="bf16")
    A, B, _ = gen.make_inputs(w, "cuda", seed=5)
    C = torch.empty((n, n // 8), dtype=torch.bfloat16, device="cuda")
    ready = torch.ones((P, (n // P) // chunk_rows), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    call = pk.BoundAgGemm(A, ready, B, C, err, n, n // 8, n, P, rank, chunk_rows, 1)
    ms, _ = time_steps(lambda i: call(), 1, warmup, steps, torch)
    assert int(err.item()) == 0
    g = pk.BoundCall(A, B, None, None, C, None, n, n // 8, n, P, 0, 0, 0, 1, gemm_only=True)
    g_ms, _ = time_steps(lambda i: g(), 1, warmup, steps, torch)
    flops = 2.0 * n * (n // 8) * n
    return {"M": n, "N": n // 8, "K": n, "P": P, "rank": rank, "chunk_rows": chunk_rows,
            "tile_order": 1, "kernel_ms": round(ms, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "gemm_only_kernel_ms": round(g_ms, 4)}


def measure_intercu(w, args, torch, gen, pk, steps, warmup, counts=(8, 16, 32, 64)):
    """The inter-CU schedule on the same share: one launch computes the share
    on CUs - n workgroups while n communicator workgroups move every send
    chunk into staging buffers; timed back to back for each n (the ready
    words count calls, so each launch moves the call it makes)."""
    s = BufferSet(w, 17, w.chunk_rows, torch, gen, pk)
    n = (w.P - 1) * (w.S // w.chunk_rows)
    dest = torch.empty_like(s.send)
    status = torch.zeros(n, dtype=torch.int32, device="cuda")
    out_bf16 = 1 if w.out_dtype == "bf16" else 0
    res = {}
    calls = 0
    for nc in counts:
        call = pk.BoundInterCU(s.A, s.B, s.peers, s.send, s.out, s.flags, dest, status, w.M, w.N,
                               w.K, w.P, w.rank, w.chunk_rows, w.tile_order, out_bf16, calls + 1,
                               nc)

        def step(i):
            nonlocal calls
            call()
            call.next()
            calls += 1
        ms, _ = time_steps(step, 1, warmup, steps, torch)
        call.check()   # raises if a communicator gave up on a chunk
        res[str(nc)] = round(ms * 1e3, 2)
    assert torch.equal(dest.view(torch.int16), s.send.view(torch.int16))
    best = min(res, key=res.get)
    return {"us_per_call_by_comm_cus": res, "best_comm_cus": int(best),
            "copy_gbps_at_best": round(2 * (w.P - 1) * w.S * w.N * 2 / (res[best] * 1e-6) / 1e9, 1)}


def torch_mm_ms(w, torch, gen, steps=5, warmup=2):
    """torch.mm (hipBLASLt) on the same bf16 GEMM: run only, as a reference."""
    A, B, _ = gen.make_inputs(gen.Workload(w.name, P=1, rank=0, M=w.M, N=w.N, K=w.K,
                                           chunk_rows=0, ab_dist=w.ab_dist, peer_dist="normal",
                                           out_dtype="bf16"), "cuda", seed=3)
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    ms, _ = time_steps(lambda i: torch.mm(A, B, out=C), 1, warmup, steps, torch)
    return round(ms, 4)


def measure_consumer(w, args, torch, gen, pk, reps=20, consumer_wgs=16):
    """The chunk consumer beside the producer on the same share.

    The producer runs on CUs - consumer_wgs workgroups.  Timed: the producer
    alone, then the producer with the consumer on a second stream (copying
    every chunk into staging buffers as its ready word rises), both as
    back-to-back repetitions bracketed by events.  Flag latency is the
    consumer's clock when it saw a word minus the producer's clock when it
    raised it (100 MHz device clock), over the chunks of the last repetition.
    """
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = BufferSet(w, 17, w.chunk_rows, torch, gen, pk)
    n = (w.P - 1) * (w.S // w.chunk_rows)
    dest = torch.empty_like(s.send)
    status = torch.zeros(n, dtype=torch.int32, device="cuda")
    observed = torch.zeros(n, dtype=torch.int64, device="cuda")
    clock = torch.zeros(n, dtype=torch.int64, device="cuda")
    out_bf16 = 1 if w.out_dtype == "bf16" else 0
    sp, sc = torch.cuda.Stream(), torch.cuda.Stream()
    prod = pk.BoundCall(s.A, s.B, s.peers, s.send, s.out, s.flags, w.M, w.N, w.K, w.P, w.rank,
                        w.chunk_rows, w.tile_order, out_bf16,
                        max_workgroups=max(cus - consumer_wgs, 1), ready_clock=clock, stream=sp)
    calls = 0

    def run(with_consumer, k):
        nonlocal calls
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(sp)
        sc.wait_event(t0)
        for _ in range(k):
            prod()
            calls += 1
            if with_consumer:
                # consumer n may start before producer call n; it waits for
                # ready words of n, and the next producer call waits for it
                # (the send buffers are reused)
                pk.pk_rs_consume(s.flags, s.send, dest, w.M, w.N, w.P, w.chunk_rows, calls,
                                 status, observed, spin_limit=1 << 16,
                                 max_workgroups=consumer_wgs, stream=sc)
                sp.wait_stream(sc)
        t1.record(sp)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / k

    run(False, 3)
    run(True, 3)
    alone = run(False, reps)
    both = run(True, reps)
    st = status.cpu()
    assert int(st.abs().max()) == 0, "the consumer timed out on a chunk"
    assert torch.equal(dest.view(torch.int16), s.send.view(torch.int16))
    lat = ((observed - clock).double() / 100.0).cpu()      # us
    return {"consumer_workgroups": consumer_wgs, "producer_workgroups": max(cus - consumer_wgs, 1),
            "producer_alone_us": round(alone * 1e3, 2),
            "producer_and_consumer_us": round(both * 1e3, 2),
            "copy_gbps": round(2 * (w.P - 1) * w.S * w.N * 2 / (both * 1e-3) / 1e9, 1),
            "flag_latency_us": {"median": round(float(lat.median()), 2),
                                "max": round(float(lat.max()), 2),
                                "min": round(float(lat.min()), 2)}}


def timeline_study(w, args, torch, gen, pk):
    """Per-workgroup phase record of the timing build of the library (the
    same sources compiled with PK_TIMELINE): each workgroup's CU placement
    and the 100 MHz device clock at each phase boundary (1 first stage
    landed, 2 main loop done, 3 epilogue done, 4 ready words raised), over
    `steps` launches back to back on rotating buffer sets.  Workgroups are
    grouped by their sequence of phases (their role in the schedule); the
    line reports the median time of each phase from the launch's first
    workgroup start, and how the workgroups shared the CUs."""
    import numpy as np
    pk.use_library(pk.TIMELINE_LIB_NAME)
    chunk = args.chunk_rows or w.chunk_rows
    order = w.tile_order if args.tile_order is None else args.tile_order
    set_bytes = w.algorithmic_bytes()
    n_sets = max(2, min(8, math.ceil(1.2 * MALL_BYTES / set_bytes))) if set_bytes < 2 * MALL_BYTES else 1
    sets = [BufferSet(w, 17 * i, chunk, torch, gen, pk) for i in range(n_sets)]
    out_bf16 = 1 if w.out_dtype == "bf16" else 0
    opts = dict(config=args.config, max_workgroups=args.max_workgroups, group_n=args.group_n,
                store_policy=args.store_policy, owned_split=args.owned_split)
    words = pk.TIMELINE_BYTES // 8
    tls = [torch.zeros(words, dtype=torch.int64, device="cuda") for _ in range(args.steps)]
    scratch = torch.zeros(words, dtype=torch.int64, device="cuda")

    def call(i, tl):
        s = sets[i % n_sets]
        return pk.BoundCall(s.A, s.B, s.peers, s.send, s.out, s.flags, w.M, w.N, w.K, w.P, w.rank,
                            chunk, order, out_bf16, timeline=tl, **opts)
    warm = [call(i, scratch) for i in range(n_sets)]
    for i in range(args.warmup):
        warm[i % n_sets]()
    steps = [call(args.warmup + i, tls[i]) for i in range(args.steps)]
    torch.cuda.synchronize()
    for c in steps:
        c()
    torch.cuda.synchronize()
    groups = {}
    spans, placement = [], None
    mask56 = (1 << 56) - 1
    for tl in tls:
        t = tl.cpu().numpy().view(np.uint64).reshape(pk.TIMELINE_WORKGROUPS, pk.TIMELINE_SLOTS)
        live = np.nonzero(t[:, 1])[0]
        t0 = int(t[live, 1].min())
        end = t0
        for b in live:
            marks = [int(m) for m in t[b, 2:] if m]
            kinds = tuple(m >> 56 for m in marks)
            times = [((m & mask56) - t0) / 100.0 for m in marks]
            g = groups.setdefault(kinds, {"workgroups": 0, "start": [], "times": []})
            g["workgroups"] += 1
            g["start"].append((int(t[b, 1]) - t0) / 100.0)
            g["times"].append(times)
            if marks:
                end = max(end, marks[-1] & mask56)
        spans.append((end - t0) / 100.0)
        if placement is None:
            hw = t[live, 0]
            cu = [(int(h >> 32), int((h >> 13) & 7), int((h >> 8) & 15)) for h in hw]
            per_cu = {}
            for b, c in zip(live, cu):
                per_cu.setdefault(c, []).append(int(b))
            grid = len(live)
            mixed = sum(1 for v in per_cu.values()
                        if any(b < grid // 2 for b in v) and any(b >= grid // 2 for b in v))
            placement = {"workgroups": grid, "cus_used": len(per_cu),
                         "workgroups_per_cu": {str(k): sum(1 for v in per_cu.values() if len(v) == k)
                                               for k in sorted({len(v) for v in per_cu.values()})},
                         "cus_with_both_halves": mixed}
    roles = []
    names = {1: "stage", 2: "main", 3: "epilogue", 4: "signal"}
    for kinds, g in sorted(groups.items(), key=lambda kv: -kv[1]["workgroups"]):
        med = np.median(np.array(g["times"]), axis=0) if g["times"] and kinds else []
        roles.append({"phases": "-".join(names.get(k, str(k)) for k in kinds),
                      "workgroups_per_launch": round(g["workgroups"] / len(tls), 1),
                      "start_us": round(float(np.median(g["start"])), 2),
                      "phase_end_us": [round(float(x), 2) for x in med]})
    pk.use_library(pk.LIB_NAME)
    return {"workload": w.name, "config": args.config, "launches": len(tls),
            "span_us_median": round(float(np.median(spans)), 2), "placement": placement,
            "roles": roles}


def source_digest():
    """sha256 over the HIP sources of the library (the kernel the counters saw)."""
    d = os.path.join(ROOT, "gemm_reduce_scatter_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_for(w):
    """Measured HBM bytes per launch of the fused kernel on workload w, or None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.txt")
    try:
        with open(path) as f:
            rec = json.loads(f.read())
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest():
        return None
    e = rec.get("workloads", {}).get(w.name)
    if not e:
        return None
    return int(round(e["fetch_kib"] * 1024 * rec["copy_fetch_factor"]
                     + e["write_kib"] * 1024 * rec["copy_write_factor"]))


def copy_calibration(torch):
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "calls": 5}), flush=True)


TRAFFIC_CMD = ("rocprofv3 --pmc {counter} -f csv -d <DIR>/<workload>_{kind} -o p -- python3 "
               "bench.py --workload <workload> --steps 5 --warmup 2 --no-secondary "
               "--no-cpu-baseline --no-gemm-only --no-push --no-consumer --no-ag-gemm --no-reduce")
COPY_CMD = "rocprofv3 --pmc {counter} -f csv -d <DIR>/copy_{kind} -o p -- python3 bench.py --copy-calibration"


def write_traffic(d):
    """profiles/pmc_traffic.txt from rocprofv3 counter runs under `d`: per
    workload the median over the fused kernel's dispatches of FETCH_SIZE and
    WRITE_SIZE (KiB), and the factors that make the counters read the bytes
    of a plain 512 MiB device copy (one dispatch of the copy kernel moves
    512 MiB each way)."""
    import csv
    import glob
    import statistics

    def per_dispatch(sub, counter, kernel_part):
        files = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        vals = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter and kernel_part in r["Kernel_Name"]:
                    key = int(r["Dispatch_Id"])
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return sorted(vals.values())

    copy_kib = 512 * 1024
    cf = statistics.median(per_dispatch("copy_fetch", "FETCH_SIZE", "opy"))
    cw = statistics.median(per_dispatch("copy_write", "WRITE_SIZE", "opy"))
    rec = {"source_sha256": source_digest(),
           "what": "fused kernel HBM traffic per launch: median over dispatches of rocprofv3 "
                   "FETCH_SIZE / WRITE_SIZE (KiB), scaled by copy_*_factor = 524288 KiB / what "
                   "the counter reads for one 512 MiB device copy",
           "copy_fetch_factor": round(copy_kib / cf, 4), "copy_write_factor": round(copy_kib / cw, 4),
           "commands": {"workload": TRAFFIC_CMD, "copy": COPY_CMD,
                        "summary": "python bench.py --write-traffic <DIR>"},
           "workloads": {}}
    for sub in sorted(os.listdir(d)):
        if not sub.endswith("_fetch") or sub.startswith("copy"):
            continue
        name = sub[:-len("_fetch")]
        fe = per_dispatch(sub, "FETCH_SIZE", "pk_gemm_rs_fused")
        wr = per_dispatch(name + "_write", "WRITE_SIZE", "pk_gemm_rs_fused")
        if fe and wr:
            rec["workloads"][name] = {"fetch_kib": round(statistics.median(fe), 1),
                                      "write_kib": round(statistics.median(wr), 1),
                                      "dispatches": [len(fe), len(wr)]}
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.txt"), "w") as f:
        f.write(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec), flush=True)


def roofline_of(w, kernel_ms, metrics):
    if w.flops() / w.algorithmic_bytes() > metrics.PEAK_BF16_DENSE_FLOPS / metrics.PEAK_HBM_BYTES:
        ach = w.flops() / (kernel_ms * 1e-3) / 1e12
        peak = metrics.PEAK_BF16_DENSE_FLOPS / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": traffic_for(w)}
    ach = w.algorithmic_bytes() / (kernel_ms * 1e-3) / 1e9
    peak = metrics.PEAK_HBM_BYTES / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": peak, "unit": "GB/s",
            "frac": round(ach / peak, 4), "traffic": traffic_for(w)}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count()]))
    except Exception:
        return int(os.cpu_count())


def cpu_baseline(w, gen, torch, unit, rows_per_shard=None, budget_s=12.0):
    """The fp64 oracle (oracle.gemm_rs_oracle as it is) on the host cores,
    called repeatedly until ``budget_s`` has passed.

    With ``rows_per_shard`` None it runs the whole share.  Otherwise it runs
    the share restricted to the first ``rows_per_shard`` rows of each of the P
    row shards: P * r rows of A, all of B, the same r rows of every peer slot,
    chunks of r rows.  Every row does what it does in the whole share (N dot
    products of length K, then its bf16 send rounding or its owned sum), so
    the rate carries over to the whole share.  The inputs are the share's
    generator output (made on the GPU); only the block goes to the host, and
    neither that copy nor the bit extraction is timed.  ``value`` is in
    ``unit``: GB/s of the block's algorithmic bytes or TFLOP/s of its
    multiply-adds."""
    import oracle.gemm_rs_oracle as orc
    if rows_per_shard is None:
        sub = w
        A, B, peers = gen.make_inputs(w, "cpu", seed=0)
        Ab, Bb, Pb = gen.bf16_bits(A), gen.bf16_bits(B), gen.bf16_bits(peers)
        what = f"the whole {w.name} share ({w.M}x{w.N}x{w.K}, P={w.P})"
    else:
        r = rows_per_shard
        sub = w.with_(M=w.P * r, chunk_rows=r)
        dev = "cuda" if torch.cuda.is_available() else "cpu"
        A, B, peers = gen.make_inputs(w, dev, seed=0)
        rows = torch.cat([torch.arange(d * w.S, d * w.S + r) for d in range(w.P)]).to(A.device)
        Ab, Bb, Pb = gen.bf16_bits(A[rows]), gen.bf16_bits(B), gen.bf16_bits(peers[:, :r])
        what = (f"a row block of the {w.name} share ({w.M}x{w.N}x{w.K}, P={w.P}, rank {w.rank}): "
                f"the first {r} rows of each of the {w.P} shards ({sub.M}x{w.N}x{w.K}, "
                f"{w.P - 1} sent chunks and one owned sum of {r} rows each)")
    del A, B, peers
    if torch.cuda.is_available():
        torch.cuda.empty_cache()
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.gemm_rs_oracle(Ab, Bb, Pb, sub.P, sub.rank, sub.chunk_rows)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 50:
            break
    per = el / n
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    if unit == "TFLOP/s":
        value = round(sub.flops() / per / 1e12, 4)
    else:
        value = round(sub.algorithmic_bytes() / per / 1e9, 3)
    return {"value": value, "unit": unit, "cores": _blas_threads(), "kind": "oracle",
            "cpu_model": model,
            "sample": f"{n} oracle calls on {what}, {per:.3f} s each, fp64 numpy/OpenBLAS",
            "tflops_fp64": round(sub.flops() / per / 1e12, 4),
            "gbps": round(sub.algorithmic_bytes() / per / 1e9, 3)}


def measure_secondary(w, args, torch, gen, pk, metrics, steps, warmup=3):
    """One of the 32768-wide shares, timed like the default share (``steps``
    back-to-back launches on one buffer set, which is larger than the
    last-level cache).  A workload with sweep points (chunk_rows x tile order)
    is first timed at every point; the best point is then timed again with
    everything else, so the reported time is not the minimum of the sweep."""
    a = argparse.Namespace(**{**vars(args), "chunk_rows": None, "tile_order": None})
    chunk = order = None
    sweep = None
    if w.sweep_chunk_rows:
        sweep = []
        for c in w.sweep_chunk_rows:
            for o in (0, 1, 2):
                r = measure(w, a, torch, gen, pk, metrics, steps, warmup, rotate=False,
                            gemm_only=False, tile_order=o, chunk_rows=c)
                sweep.append({"chunk_rows": c, "tile_order": o,
                              "kernel_ms": round(r["kernel_ms"], 4)})
        best = min(sweep, key=lambda p: p["kernel_ms"])
        chunk, order = best["chunk_rows"], best["tile_order"]
    r = measure(w, a, torch, gen, pk, metrics, steps, warmup, rotate=False,
                gemm_only=not args.no_gemm_only, tile_order=order, chunk_rows=chunk,
                reduce_counts=() if args.no_reduce else (16, 32),
                # owned tiles wait for the reduction: an order that reaches
                # them late (row-major; the owned shard is rank's)
                reduce_order=0)
    roof = roofline_of(w, r["kernel_ms"], metrics)
    sec = {"workload": w.name, "P": w.P, "rank": w.rank, "M": w.M, "N": w.N, "K": w.K,
           "out": w.out_dtype, "chunk_rows": r["chunk_rows"], "tile_order": r["tile_order"],
           "steps": steps, "warmup": warmup, "kernel_ms": round(r["kernel_ms"], 4),
           "tflops": round(w.flops() / (r["kernel_ms"] * 1e-3) / 1e12, 2), "roofline": roof}
    if sweep is not None:
        sec["sweep"] = sweep
    if "gemm_only_kernel_ms" in r:
        sec["gemm_only_kernel_ms"] = round(r["gemm_only_kernel_ms"], 4)
        sec["exposed_fraction"] = round(r["exposed_fraction"], 4)
    if "inter_cu_reduce" in r:
        sec["inter_cu_reduce"] = r["inter_cu_reduce"]
    if not args.no_push:
        pu = measure_push(w, args, torch, gen, pk, steps, warmup)
        sec["atomic_push_kernel_ms"] = pu["kernel_ms"]
    sec["torch_mm_ms"] = torch_mm_ms(w, torch, gen, steps=steps, warmup=warmup)
    if not args.no_cpu_baseline:
        sec["cpu_baseline"] = cpu_baseline(w, gen, torch, roof["unit"], rows_per_shard=64,
                                           budget_s=6.0)
    return sec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported "
              f"(the multi-GPU exchange is not part of this library)", file=sys.stderr)
        sys.exit(2)
    import torch

    from gemm_reduce_scatter_amd import binding as pk
    from gemm_reduce_scatter_amd import inputs as gen
    from gemm_reduce_scatter_amd import metrics

    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    torch.cuda.init()
    if args.copy_calibration:
        copy_calibration(torch)
        return
    pk.load()
    w = gen.WORKLOADS[args.workload]
    if args.timeline:
        print(json.dumps(timeline_study(w, args, torch, gen, pk)), flush=True)
        return
    if args.sweep:
        w = gen.WORKLOADS["large_k"]
        for chunk in w.sweep_chunk_rows:
            for order in (0, 1, 2):
                r = measure(w, args, torch, gen, pk, metrics, max(3, args.steps // 5), 2,
                            rotate=False, gemm_only=False, tile_order=order, chunk_rows=chunk)
                print(json.dumps({"workload": w.name, "chunk_rows": chunk, "tile_order": order,
                                  "kernel_ms": round(r["kernel_ms"], 4),
                                  "tflops": round(w.flops() / r["kernel_ms"] / 1e9, 1)}),
                      flush=True)
        return

    # 0 reduction workgroups: the reduction runs in the background of the
    # main loops, which needs P = 8 and a grid that holds every 256 x 256 tile
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    bg = w.P == 8 and 8 * math.ceil(w.S / 256) * math.ceil(w.N / 256) <= cus
    r = measure(w, args, torch, gen, pk, metrics, args.steps, args.warmup,
                gemm_only=not args.no_gemm_only,
                reduce_counts=() if args.no_reduce else ((0,) if bg else ()) + (8, 16, 32, 64))
    roof = roofline_of(w, r["kernel_ms"], metrics)
    cfg_id = args.config or pk.pk_select_config(w.M, w.N, w.K, w.P)
    if roof["bound"] == "hbm":
        value = w.algorithmic_bytes() / (r["ms_per_step"] * 1e-3) / 1e9
        unit = "GB/s"
    else:
        value = w.flops() / (r["ms_per_step"] * 1e-3) / 1e12
        unit = "TFLOP/s"
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "P": w.P, "rank": w.rank, "M": w.M, "N": w.N, "K": w.K,
                   "chunk_rows": r["chunk_rows"], "tile_order": r["tile_order"],
                   "out": w.out_dtype, "tile_config": pk.pk_config_info(cfg_id),
                   "buffer_sets": r["n_sets"]},
        "roofline": roof,
        "kernel_ms": round(r["kernel_ms"], 5),
        "tflops": round(w.flops() / (r["kernel_ms"] * 1e-3) / 1e12, 2),
        "epilogue_gbps": round(w.epilogue_bytes() / (r["kernel_ms"] * 1e-3) / 1e9, 1),
    }
    if "gemm_only_kernel_ms" in r:
        line["gemm_only_kernel_ms"] = round(r["gemm_only_kernel_ms"], 5)
        line["exposed_fraction"] = round(r["exposed_fraction"], 4)
        line["torch_mm_ms"] = torch_mm_ms(w, torch, gen, steps=max(5, min(args.steps, 50)))
    if "inter_cu_reduce" in r:
        line["inter_cu_reduce"] = r["inter_cu_reduce"]
    if not args.no_secondary:
        # at least 20 timed launches each (a compute-bound launch is 4-14 ms)
        sec_steps = max(20, args.steps // 10)
        secs = [measure_secondary(gen.WORKLOADS[name], args, torch, gen, pk, metrics, sec_steps)
                for name in ("near_threshold", "compute_bound", "large_k")
                if name != args.workload]
        if secs:
            line["secondary"] = secs
    if not args.no_push:
        pu = measure_push(w, args, torch, gen, pk, args.steps, args.warmup)
        pu["vs_staged"] = round(pu["kernel_ms"] / r["kernel_ms"], 3)
        line["atomic_push"] = pu
    if not args.no_consumer and w.P > 1:
        line["chunk_consumer"] = measure_consumer(w, args, torch, gen, pk)
    if not args.no_consumer and w.P > 1:
        line["inter_cu"] = measure_intercu(w, args, torch, gen, pk, args.steps, args.warmup)
    if not args.no_ag_gemm:
        line["ag_gemm"] = measure_ag_gemm(torch, gen, pk, max(20, args.steps // 10), 3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, gen, torch, unit)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
