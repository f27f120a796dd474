"""Benchmark of the Reverse All2All combine on one MI355X.

One step = one whole combine: the signal reset, then the signal-pipelined
persistent kernel (the library default: direct mode with row units on this
shape), over the EP-combine
workload: W=8 simulated ranks (slices of one symmetric heap), S=512 tokens,
H=16 heads, D=128, bf16 values uniform(-1, 1) from seed 0, 64 x 1 x 128
signal tiles with ADD-to-W tile signals.  Inputs are resident in HBM before
timing starts.  So that the 256 MiB working set is not served from the 256 MB
Infinity Cache, consecutive steps rotate through several in/out/signal buffer
sets.  Three ways of issuing the steps are timed, every one of which zeroes a
step's signals before any of its producers signals: in-launch (the library
default: one launch per step, whose first workgroups zero the signals),
serial (a reset launch, then the combine, on one stream) and overlapped (a
step's reset launch on a side stream while the previous step's combine runs
-- it touches only its own set's signals -- and the combine waiting for it);
`value` is the fastest, and all three are reported.

Prints one JSON line: metric and value (GB/s of algorithmic bytes: every input
element read once and every output element written once, per step), the
roofline of the persistent kernel (its average launch duration: HIP events on
the launch stream around the in-launch timed region, one launch per step, no
events between launches), and for context per-source pieces, the staged mode,
the two-phase variant, a
plain copy of the same bytes with the library's put kernel, the bulk mode
(two-phase layout with per-(S-block, sender) signals), the pull mode, the forward
All2All (dispatch, the combine's inverse map) on the same buffers, and the CPU
oracle's rate on the host.

``--legs main`` runs only the timed combine (for counter runs under rocprofv3).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "ep_combine_w8_s512_h16_d128_bf16"
HBM_PEAK_GBS = 8000.0
# what ra2a_rev_all2all_plan reports as the mode a combine resolves to
MODE_NAMES = {1: "per-source pieces", 2: "staged", 3: "bulk", 4: "pull",
              5: "row units (whole out_j rows, all sources)"}
NSETS = 6
BIG_ALIGN = 2 << 20  # placement of the combine's inputs and outputs in a slice


def kernel_label(mode):
    """The dominant kernel of a combine leg, named with the mode its plan resolves to."""
    return (f"rev_a2a_pipelined_kernel (direct mode: {MODE_NAMES.get(mode, '?')}, "
            "write-through stores)")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_rev_a2a_pipelined_direct_ep_combine_w8.json")
TRAFFIC_FILE_MOE = os.path.join(ROOT, "profiles", "traffic_rev_a2a_pipelined_direct_moe_combine_w8.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the sources the persistent kernel is compiled from and of the host
    code that plans its launches (piece shapes, schedule)."""
    h = hashlib.sha256()
    for f in ("combine_kernels.hip", "combine_geom.h", "device.h", "common.h", "queue.h", "api.hip"):
        with open(os.path.join(ROOT, "moe_all2all_combine_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch of the persistent kernel from the committed rocprofv3
    counter runs, if they were taken on the current kernel source; else None."""
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(wl, ins, run_s=2.5):
    """The CPU oracle as it stands on the host cores: repeated full combines of the
    workload, timed on one thread and on every core this process may use (the
    combine split over (destination, token range) with the oracle's row-range
    entry; ctypes releases the GIL during each C call), median of 3 runs each;
    plus the fp64 GEMM oracle (numpy on all cores) on a bounded sample of the
    AllGather+GEMM workload."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    from oracle import gemm

    W, S = wl.W, wl.S
    nthreads = len(os.sched_getaffinity(0))
    outs = [np.empty((S, wl.H * W, wl.D), dtype=ins[0].dtype) for _ in range(W)]
    per = max(1, -(-nthreads // W))  # token ranges per destination
    cuts = [S * k // per for k in range(per + 1)]
    tasks = [(j, cuts[k], cuts[k + 1]) for j in range(W) for k in range(per)]

    def one_thread():
        for j in range(W):
            oracle.combine_dest_rows(ins, outs[j], j, 0, S)

    pool = cf.ThreadPoolExecutor(max_workers=nthreads)

    def all_threads():
        list(pool.map(lambda t: oracle.combine_dest_rows(ins, outs[t[0]], *t), tasks))

    def rate(fn):
        t0 = time.perf_counter()
        fn()
        one = time.perf_counter() - t0
        reps = max(1, int(run_s / max(one, 1e-6)))
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            for _ in range(reps):
                fn()
            runs.append(wl.algorithmic_bytes * reps / (time.perf_counter() - t0) / 1e9)
        return float(np.median(runs)), reps

    v1, r1 = rate(one_thread)
    vn, rn = rate(all_threads)
    pool.shutdown()
    ok = all(outs[j].tobytes() == oracle.combine_dest(ins, j).tobytes() for j in range(W))
    # the fp64 GEMM oracle on the first 256 rows of every shard of the AllGather+GEMM
    import synthgen
    g = synthgen.AG_GEMM
    shards, b = synthgen.make_ag_gemm_inputs(g, m_local=256)
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        gemm.ag_gemm_ref(shards, b)
        runs.append(2.0 * g.W * 256 * g.K * g.N / (time.perf_counter() - t0) / 1e9)
    return {"value": round(vn, 3), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{rn} full combines of the {wl.name} workload per run "
                      f"({wl.algorithmic_bytes >> 20} MiB moved each), split over {len(tasks)} "
                      f"(destination, token range) tasks on {nthreads} threads; median of 3 runs",
            "one_thread": {"value": round(v1, 3), "unit": "GB/s", "cores": 1,
                           "sample": f"{r1} full combines per run, median of 3 runs"},
            "parity_with_oracle": ok,
            "gemm_fp64": {"value": round(float(np.median(runs)), 2), "unit": "GFLOP/s",
                          "cores": nthreads, "sample": f"{g.name} restricted to 256 rows per shard "
                          f"({g.W * 256} x {g.K} x {g.N}), numpy float64, median of 3 runs"},
            "host": host_cpu()}


def host_cpu():
    """The host the CPU baseline ran on: the CPU model string and its family /
    model / stepping numbers (/proc/cpuinfo), cores this process may use, cores
    online."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                k, _, v = line.partition(":")
                k = k.strip()
                if k in ("model name", "cpu family", "model", "stepping", "cpu MHz") and k not in info:
                    info[k] = v.strip()
                if not line.strip() and info:
                    break
    except OSError:
        pass
    return {"cpu_model": info.get("model name", "unknown"),
            "cpu_family_model_stepping": [info.get("cpu family"), info.get("model"), info.get("stepping")],
            "affinity": len(os.sched_getaffinity(0)), "online": os.cpu_count()}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def steady_times(fns, steps, stream, warm=12, rounds=2):
    """Milliseconds per call of each callable in `fns` (name -> fn) in steady state:
    every one is first called `warm` times (first calls of a library pick and load
    their kernels, and the clocks settle), then timed `rounds` times over `steps`
    calls with HIP events on `stream`, the callables taking turns; the best round
    counts."""
    import torch

    for fn in fns.values():
        for _ in range(warm):
            fn()
    torch.cuda.synchronize()
    best = {k: float("inf") for k in fns}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(rounds):
        for k, fn in fns.items():
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            best[k] = min(best[k], e0.elapsed_time(e1) / steps)
    return best


def cold_times(fns, calls, stream, flush_bytes=512 << 20):
    """Milliseconds per call of each callable with the Infinity Cache cold: before
    every call a copy of `flush_bytes` (twice the 256 MB cache) evicts what the
    previous call left there; HIP events around each call alone, the mean over
    `calls` calls (after one untimed call each)."""
    import torch

    a = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    out = {}
    for k, fn in fns.items():
        fn()
        tot = 0.0
        for _ in range(calls):
            b.copy_(a)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            tot += e0.elapsed_time(e1)
        out[k] = tot / calls
    del a, b
    return out


def ag_gemm_leg(steps):
    """The AllGather+GEMM workload (W=8 shards of 1024 x 7168 gathered, times a
    7168 x 4096 B; bf16 in, fp32 accumulation, bf16 out), for context: one call
    = B transposed into the workspace + signal reset + the persistent launch."""
    import numpy as np
    import torch

    import moe_all2all_combine_amd as ra2a
    import synthgen

    g = synthgen.AG_GEMM
    W, m, K, N, tr = g.W, g.m_local, g.K, g.N, g.tile_rows
    nsig = sum(ra2a.ag_gemm_signal_slots(W, m, tr))
    sb = m * K * 2
    heap = ra2a.SymmHeap(W, sb + W * sb + nsig * 128 + (1 << 16))
    try:
        oa, og, osg = heap.alloc(sb), heap.alloc(W * sb), heap.alloc(nsig * 128)
        gen = torch.Generator(device="cuda").manual_seed(g.seed_a)
        for w in range(W):
            heap.view(oa, (m * K,), torch.bfloat16, w).copy_(
                torch.randn(m * K, generator=gen, device="cuda") * g.std)
        b = (torch.randn(K, N, generator=gen, device="cuda") * g.std).to(torch.bfloat16)
        c = torch.empty(W * m, N, dtype=torch.bfloat16, device="cuda")
        st = torch.cuda.current_stream()

        def call():
            ra2a.ag_gemm(heap.ptr(oa), heap.ptr(og), b.data_ptr(), c.data_ptr(), heap.ptr(osg),
                         W, 0, m, K, N, tr, 0, st)

        # with B already transposed (one launch each, after a reset launch): the
        # persistent kernel's roofline
        bt = b.t().contiguous()

        def call_bt():
            ra2a.ag_gemm(heap.ptr(oa), heap.ptr(og), bt.data_ptr(), c.data_ptr(), heap.ptr(osg),
                         W, 0, m, K, N, tr, ra2a.AG_B_TRANSPOSED, st)

        # the unfused library sequence on the same inputs: gather the shards into G
        # (device copies), then the library GEMM, with B as K x N and with B given
        # transposed (N x K, a linear layer's weight layout: the library multiplies
        # by the transposed view, no copy)
        shards_t = [heap.view(oa, (m, K), torch.bfloat16, w) for w in range(W)]
        gbuf = torch.empty(W * m, K, dtype=torch.bfloat16, device="cuda")
        cl = torch.empty(W * m, N, dtype=torch.bfloat16, device="cuda")

        def lib_seq():
            for w in range(W):
                gbuf[w * m:(w + 1) * m].copy_(shards_t[w])
            torch.matmul(gbuf, b, out=cl)

        def lib_seq_bt():
            for w in range(W):
                gbuf[w * m:(w + 1) * m].copy_(shards_t[w])
            torch.mm(gbuf, bt.t(), out=cl)

        t = steady_times({"call": call, "call_bt": call_bt, "lib": lib_seq, "lib_bt": lib_seq_bt}, steps, st)
        cold = cold_times({"call_bt": call_bt, "lib_bt": lib_seq_bt}, 10, st)
        assert ra2a.check(heap.handle) == ra2a.OK, ra2a.last_error()
        ms, bt_ms, lib_ms, lib_bt_ms = t["call"], t["call_bt"], t["lib"], t["lib_bt"]
        flops = 2.0 * W * m * N * K
        tf = flops / (ms * 1e-3) / 1e12
        ktf = flops / (bt_ms * 1e-3) / 1e12
        return {"workload": g.name, "ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                "library_sequence": {"ms": round(lib_ms, 4),
                                     "TFLOP/s": round(flops / (lib_ms * 1e-3) / 1e12, 1),
                                     "what": "W shard copies into G, then torch.matmul(G, B) (bf16)"},
                "b_transposed": {"ms": round(bt_ms, 4),
                                 "what": "one call with B passed as B^T (N x K): reset + persistent launch",
                                 "library_sequence_ms": round(lib_bt_ms, 4),
                                 "library_sequence": "W shard copies into G, then torch.mm(G, B^T viewed "
                                                     "transposed) (bf16)",
                                 "cold": {"ms": round(cold["call_bt"], 4),
                                          "library_sequence_ms": round(cold["lib_bt"], 4),
                                          "what": "each call after a 512 MiB copy that evicts the "
                                                  "Infinity Cache (events around each call)"}},
                "frac_of_bf16_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "calls": steps,
                "note": "one call = B transposed into the workspace + signal reset + persistent launch; "
                        "steady state: every variant called 12 times first, then two rounds of "
                        "timed calls taking turns, the best round (HIP events)",
                "roofline": {"bound": "mfma", "achieved": round(ktf, 1),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(ktf / MFMA_BF16_PEAK_TFLOPS, 4),
                             "kernel": "ag_gemm_kernel (B passed transposed: reset + one launch per call)",
                             "ms_per_call": round(bt_ms, 4), "flop_per_launch": flops}}
    finally:
        heap.close()


def gemm_rs_leg(steps):
    """The GEMM + ReduceScatter workload (W=8 ranks, x1_r 8192 x 896, x2_r
    896 x 4096; bf16 in, fp32 partials and sums, bf16 out): one call = signal
    reset + the persistent launch; also timed with the partials rounded to bf16.  For context, the same product as a library
    sequence without overlap: W torch.mm calls (bf16 out) then a sum over the
    sources of each destination's rows."""
    import torch

    import moe_all2all_combine_amd as ra2a
    import synthgen

    g = synthgen.GEMM_RS
    W, m, K, N = g.W, g.m, g.K, g.N
    mj = m // W
    nt, nq, pbytes = ra2a.gemm_rs_sizes(W, m, K, N)  # fp32 partials: the larger area
    nsig = nt + nq
    na, nb, no = m * K * 2, N * K * 2, mj * N * 2
    heap = ra2a.SymmHeap(W, na + nb + pbytes + no + nsig * 128 + (1 << 16))
    try:
        oa, ob, op = heap.alloc(na), heap.alloc(nb), heap.alloc(pbytes)
        oo, osg = heap.alloc(no), heap.alloc(nsig * 128)
        gen = torch.Generator(device="cuda").manual_seed(g.seed_a)
        for r in range(W):
            heap.view(oa, (m, K), torch.bfloat16, r).copy_(
                torch.randn(m, K, generator=gen, device="cuda") * g.std)
            heap.view(ob, (N, K), torch.bfloat16, r).copy_(
                torch.randn(N, K, generator=gen, device="cuda") * g.std)
        st = torch.cuda.current_stream()

        def call(flags=0):
            ra2a.gemm_rs(heap.ptr(oa), heap.ptr(ob), heap.ptr(op), heap.ptr(oo), heap.ptr(osg),
                         W, m, K, N, flags, st)

        # the library sequence, on the same inputs
        x1 = [heap.view(oa, (m, K), torch.bfloat16, r) for r in range(W)]
        x2 = [heap.view(ob, (N, K), torch.bfloat16, r).t() for r in range(W)]
        part = torch.empty(W, m, N, dtype=torch.bfloat16, device="cuda")
        out = torch.empty(m, N, dtype=torch.float32, device="cuda")

        def lib():
            for r in range(W):
                torch.mm(x1[r], x2[r], out=part[r])
            torch.sum(part, dim=0, dtype=torch.float32, out=out)

        t = steady_times({"f32": call, "bf16": lambda: call(ra2a.RS_BF16_PARTIALS), "lib": lib}, steps, st)
        assert ra2a.check(heap.handle) == ra2a.OK, ra2a.last_error()
        ms, bf16p_ms, lib_ms = t["f32"], t["bf16"], t["lib"]
        flops = 2.0 * W * m * N * K
        tf = flops / (ms * 1e-3) / 1e12
        return {"workload": g.name, "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "calls": steps,
                "note": "one call = signal reset + persistent launch; fp32 partials; steady state: "
                        "every variant called 12 times first, then two rounds of timed calls taking "
                        "turns, the best round (HIP events)",
                "bf16_partials": {"ms": round(bf16p_ms, 4),
                                  "TFLOP/s": round(flops / (bf16p_ms * 1e-3) / 1e12, 1)},
                "library_sequence": {"ms": round(lib_ms, 4),
                                     "TFLOP/s": round(flops / (lib_ms * 1e-3) / 1e12, 1),
                                     "what": "W torch.mm (bf16 out) + fp32 sum over sources",
                                     "same_arithmetic_as": "bf16_partials (each rank's product "
                                                           "rounded to bf16, summed in fp32)",
                                     "bf16_partials_over_library": round(bf16p_ms / lib_ms, 4)},
                "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                             "kernel": "gemm_rs_kernel (reset + one launch per call)",
                             "ms_per_call": round(ms, 4), "flop_per_launch": flops}}
    finally:
        heap.close()


def alltoallv_leg(steps):
    """The variable-size AllToAll on the MoE-shaped workload (W=8, 32768 rows of
    14336 bytes per rank, Dirichlet-multinomial routing counts; random bytes): one
    call = signal reset + the persistent launch.  Algorithmic bytes = every sent
    row read once and written once."""
    import numpy as np
    import torch

    import moe_all2all_combine_amd as ra2a
    import synthgen

    g = synthgen.ALLTOALLV
    W, rows, rb = g.W, g.rows, g.row_bytes
    c = synthgen.make_alltoallv_counts(W, rows, g.seed, g.alpha)
    out_rows = int(c.sum(axis=0).max())
    nsig = ra2a.alltoallv_signal_slots(W)
    heap = ra2a.SymmHeap(W, rows * rb + out_rows * rb + (2 * W + 1) * 8 + nsig * 128 + (1 << 16))
    try:
        oi, oo = heap.alloc(rows * rb, 16), heap.alloc(out_rows * rb, 16)
        oc, orc, osg = heap.alloc(W * 8, 8), heap.alloc((W + 1) * 8, 8), heap.alloc(nsig * 128)
        gen = torch.Generator(device="cuda").manual_seed(g.seed)
        for r in range(W):
            heap.view(oi, (rows, rb), torch.uint8, r).copy_(
                torch.randint(0, 256, (rows, rb), generator=gen, device="cuda", dtype=torch.uint8))
            heap.view(oc, (W,), torch.int64, r).copy_(torch.from_numpy(np.ascontiguousarray(c[r])))
        st = torch.cuda.current_stream()

        def call():
            ra2a.alltoallv(heap.ptr(oi), heap.ptr(oc), heap.ptr(oo), heap.ptr(orc), heap.ptr(osg), W,
                           rb, rows, out_rows, 0, 0, st)

        for _ in range(2):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(steps):
            call()
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        assert ra2a.check(heap.handle) == ra2a.OK, ra2a.last_error()
        # parity: out_j is the rank-order concatenation of the segments for j
        # (segment offsets from prefix sums of the counts), compared on the device
        so = np.cumsum(c, axis=1) - c
        ok = True
        for j in range(W):
            o = heap.view(oo, (out_rows, rb), torch.uint8, j)
            at = 0
            for r in range(W):
                n = int(c[r, j])
                seg = heap.view(oi, (rows, rb), torch.uint8, r)[int(so[r, j]):int(so[r, j]) + n]
                ok = ok and torch.equal(o[at:at + n], seg)
                at += n
            ok = ok and bool((heap.view(orc, (W + 1,), torch.int64, j).cpu().numpy()
                              == np.append(c[:, j], c[:, j].sum())).all())
        alg = 2 * int(c.sum()) * rb
        gbs = alg / (ms * 1e-3) / 1e9
        return {"workload": g.name, "ms": round(ms, 4), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "parity": ok, "calls": steps,
                "algorithmic_bytes": alg,
                "note": "one call = signal reset + persistent launch (metadata exchange + chunked push)"}
    finally:
        heap.close()


def put_calibration(heap, src_off, dst_off, nbytes, calls=8):
    """Counter calibration: the library's put kernel copying a known `nbytes`
    (slice 0 -> slice 0), so that a counter pass over the same process reads
    what FETCH_SIZE / WRITE_SIZE report for exactly nbytes read and written."""
    import torch

    import moe_all2all_combine_amd as ra2a

    for _ in range(calls):
        ra2a.put(heap.handle, heap.ptr(dst_off), heap.ptr(src_off), nbytes, 0,
                 torch.cuda.current_stream())
    torch.cuda.synchronize()


def staged_ring_leg(steps, warmup, tile_s, ring):
    """The staged mode on the EP-combine workload with a given tile_s and ring
    depth (S-blocks), over the rotated buffer sets, for counter runs on how much
    of the staging reaches HBM: one launch per step (reset launch + combine),
    parity of the last step, then the put-kernel copy of one rank's bytes that
    calibrates FETCH_SIZE / WRITE_SIZE."""
    import torch

    import moe_all2all_combine_amd as ra2a
    import synthgen

    wl = synthgen.WORKLOADS[WORKLOAD]
    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    proto = ra2a.PROTO_SET if wl.protocol == synthgen.PROTOCOL_SET else ra2a.PROTO_ADD
    o = ra2a.Opts(tile_s=tile_s, tile_h=wl.tile_h, tile_d=wl.tile_d, protocol=proto,
                  mode=ra2a.MODE_STAGED, ring=ring)
    nb = wl.bytes_per_rank
    nsig = sum(ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, o))
    work = ra2a.rev_all2all_workspace_bytes(W, S, H, D, wl.dtype, o)
    heap = ra2a.SymmHeap(W, NSETS * (2 * nb + nsig * 128 + 4096 + 2 * BIG_ALIGN) + work + (4 << 20))
    try:
        sets = [(heap.alloc(nb, BIG_ALIGN), heap.alloc(nb, BIG_ALIGN), heap.alloc(nsig * 128))
                for _ in range(NSETS)]
        for oi, _, _ in sets:
            device_inputs(heap, oi, wl, torch.int16)
        st = torch.cuda.current_stream()

        def step(k):
            oi, oo, osg = sets[k % NSETS]
            ra2a.rev_all2all_ex(heap.ptr(oi), heap.ptr(oo), heap.ptr(osg), W, S, H, D, wl.dtype, o, st)

        for k in range(warmup):
            step(k)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for k in range(steps):
            step(k)
        e1.record(st)
        torch.cuda.synchronize()
        assert ra2a.check(heap.handle) == ra2a.OK, ra2a.last_error()
        ms = e0.elapsed_time(e1) / steps
        oi, oo, _ = sets[(steps - 1) % NSETS]
        ok = all(torch.equal(heap.view(oo, (S, W, H, D), torch.int16, j)[:, r],
                             heap.view(oi, (W, S, H, D), torch.int16, r)[j])
                 for j in range(W) for r in range(W))
        put_calibration(heap, sets[0][0], sets[0][1], nb)
        gbs = wl.algorithmic_bytes / (ms * 1e-3) / 1e9
        return {"workload": wl.name, "tile_s": tile_s, "ring": ring, "ring_bytes_per_slice": work,
                "ms_per_step": round(ms, 5), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / 8000, 2), "parity": ok,
                "step": "reset launch + staged combine", "calibration_put_bytes": nb}
    finally:
        heap.close()


def device_inputs(heap, off, wl, bits):
    """The workload's inputs generated on the device from its seed: the same
    distribution as synthgen's recipe (uniform(-1, 1) or normal(0, std), then
    rounded to the element type), from torch's device generator, so that the
    multi-GiB workloads need no host generation."""
    import torch

    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[wl.dtype]
    for r in range(wl.W):
        v = heap.view(off, (wl.S * wl.W, wl.H, wl.D), dt, r)
        if wl.dist == "normal":
            v.copy_(torch.randn(v.shape, generator=gen, device="cuda") * wl.std)
        else:
            v.copy_(torch.rand(v.shape, generator=gen, device="cuda") * 2 - 1)


def combine_views_match(heap, oi, oo, wl, bits):
    """The definition out_j[s, r*H + h, d] = in_r[j*S + s, h, d], checked on the
    device as bits with torch views."""
    import torch

    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    return all(torch.equal(heap.view(oo, (S, W, H, D), bits, j)[:, r],
                           heap.view(oi, (W, S, H, D), bits, r)[j])
               for j in range(W) for r in range(W))


def moe_leg(steps, profile=False):
    """The MoE-combine-shaped workload (W=8, S=4096, H=1, D=7168 bf16, 32-token
    tiles, ADD): one step = one combine with the library defaults (in-launch
    reset, one launch), on one buffer set (7.5 GB, far beyond the 256 MB MALL).
    Its own roofline: algorithmic bytes / the launch's average duration (HIP
    events on the launch stream around the timed steps).  Row units and whole-
    tile pieces for context."""
    import torch

    import moe_all2all_combine_amd as ra2a
    import synthgen

    wl = synthgen.WORKLOADS["moe_combine_w8_s4096_h1_d7168_bf16"]
    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    tiles = dict(tile_s=wl.tile_s, tile_h=wl.tile_h, tile_d=wl.tile_d, protocol=ra2a.PROTO_ADD)
    variants = {"default": ra2a.Opts(**tiles), "rows": ra2a.Opts(mode=ra2a.MODE_ROWS, **tiles),
                "whole_tile_pieces": ra2a.Opts(piece_rows=wl.tile_s, **tiles)}
    if profile:  # counter runs: the default variant only, and a calibration copy
        variants = {"default": variants["default"]}
    nsig = max(sum(ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, o)) for o in variants.values())
    nb = wl.bytes_per_rank
    heap = ra2a.SymmHeap(W, 2 * nb + nsig * 128 + (4 << 20))
    try:
        oi, oo, osg = heap.alloc(nb), heap.alloc(nb), heap.alloc(nsig * 128)
        bits = torch.int16
        device_inputs(heap, oi, wl, bits)
        st = torch.cuda.current_stream()
        if profile:
            put_calibration(heap, oi, oo, 16 << 20)
        res = {}
        for name, o in variants.items():
            def call():
                ra2a.rev_all2all_ex(heap.ptr(oi), heap.ptr(oo), heap.ptr(osg), W, S, H, D, wl.dtype, o,
                                    st)
            for _ in range(2):
                call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(st)
            for _ in range(steps):
                call()
            e1.record(st)
            torch.cuda.synchronize()
            assert ra2a.check(heap.handle) == ra2a.OK, ra2a.last_error()
            ms = e0.elapsed_time(e1) / steps
            # parity of this variant: output poisoned, one more call, the definition
            for j in range(W):
                heap.view(oo, (nb,), torch.uint8, j).fill_(0xA5)
            call()
            torch.cuda.synchronize()
            ok = ra2a.check(heap.handle) == ra2a.OK and combine_views_match(heap, oi, oo, wl, bits)
            res[name] = (ms, ok)
        alg = wl.algorithmic_bytes
        ms, ok = res["default"]
        gbs = alg / (ms * 1e-3) / 1e9
        pl = ra2a.rev_all2all_plan(W, S, H, D, wl.dtype, variants["default"])
        out = {"workload": wl.name, "ms": round(ms, 4), "GB/s": round(gbs, 1),
               "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "parity": ok, "steps": steps,
               "algorithmic_bytes": alg,
               "plan": {"piece_rows": pl.piece_rows, "pieces_per_tile": pl.pieces_per_tile,
                        "pieces": pl.work_items},
               "note": "one step = one launch (in-launch reset + combine), inputs generated on the "
                       "device from seed 1 (normal(0, 1) in bf16)",
               "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                            "traffic": load_traffic(TRAFFIC_FILE_MOE),
                            "kernel": kernel_label(pl.mode), "kernel_ms": round(ms, 5)}}
        for name in [n for n in ("rows", "whole_tile_pieces") if n in res]:
            m2, ok2 = res[name]
            g2 = alg / (m2 * 1e-3) / 1e9
            out[name] = {"ms": round(m2, 4), "GB/s": round(g2, 1),
                         "pct_hbm_peak": round(100 * g2 / HBM_PEAK_GBS, 2), "parity": ok2}
        return out
    finally:
        heap.close()


def straggler_leg():
    """The straggler workload (W=16, S=2048, H=32, D=128 fp32, 64 x 1 x 128 tiles,
    SET per (tile, source)): before each of its pieces, the source slice drawn
    from seed 2 waits n0 + u ticks of the 100 MHz device clock (u uniform in
    [0, n0], SplitMix64 from seed 2).  n0 is calibrated once, here, from the
    undelayed launch: a piece then holds its workgroup for t_piece = launch time
    x workgroups / pieces on average, and n0 = t_piece / 1.5 makes the mean wait
    (1.5 n0) equal to t_piece, so a delayed slice's pieces take about twice an
    unperturbed slice's.  Then, in direct and staged mode: the launch time with
    and without the delay, and the per-tile completion times (device clock stamps,
    microseconds from the launch's first stamp) of the delayed source against the
    others -- a consumer waits tile by tile, only for its own tile's source."""
    import numpy as np
    import torch

    import moe_all2all_combine_amd as ra2a
    import synthgen

    wl = synthgen.WORKLOADS["straggler_w16_s2048_h32_d128_f32"]
    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    lag = synthgen.straggler_rank(wl)
    base = dict(tile_s=wl.tile_s, tile_h=wl.tile_h, tile_d=wl.tile_d, protocol=ra2a.PROTO_SET)
    o_st = ra2a.Opts(mode=ra2a.MODE_STAGED, consumer_split=1, **base)
    nt = ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, ra2a.Opts(**base))[0]
    nsig = max(sum(ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, o))
               for o in (ra2a.Opts(**base), o_st))
    ring = ra2a.rev_all2all_workspace_bytes(W, S, H, D, wl.dtype, o_st)
    nb = wl.bytes_per_rank
    heap = ra2a.SymmHeap(W, 2 * nb + ring + nsig * 128 + (4 << 20))
    try:
        oi, oo, osg = heap.alloc(nb), heap.alloc(nb), heap.alloc(nsig * 128)
        device_inputs(heap, oi, wl, torch.int32)
        stamps = torch.zeros(W * nt, dtype=torch.int64, device="cuda")
        st = torch.cuda.current_stream()

        def opts(n0, mode):
            return ra2a.Opts(mode=mode, consumer_split=1, straggler_rank=lag if n0 else -1,
                             straggler_delay=n0, straggler_seed=wl.seed,
                             timestamps=stamps.data_ptr(), **base)

        def run(n0, mode=0, reps=3):
            o = opts(n0, mode)
            call = lambda: ra2a.rev_all2all_ex(heap.ptr(oi), heap.ptr(oo), heap.ptr(osg), W, S, H,
                                               D, wl.dtype, o, st)
            call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(st)
            for _ in range(reps):
                call()
            e1.record(st)
            torch.cuda.synchronize()
            assert ra2a.check(heap.handle) == ra2a.OK, ra2a.last_error()
            t = stamps.cpu().numpy().view(np.uint64).reshape(W, nt // W, W).astype(np.float64)
            t = (t - t.min()) / 100.0  # the 100 MHz device clock -> microseconds
            return e0.elapsed_time(e1) / reps, t[:, :, lag], np.delete(t, lag, axis=2)

        # calibration from the undelayed default launch
        plan = ra2a.rev_all2all_plan(W, S, H, D, wl.dtype, opts(0, 0))
        props = torch.cuda.get_device_properties(0)
        ms0, _, _ = run(0)
        wg = min(plan.work_items, props.multi_processor_count)  # one workgroup per CU (dynamic)
        t_piece_us = ms0 * 1e3 * wg / plan.work_items
        n0 = max(1, int(round(t_piece_us * 100 / 1.5)))

        def q(a):
            return {"p50": round(float(np.percentile(a, 50)), 1),
                    "p90": round(float(np.percentile(a, 90)), 1), "max": round(float(a.max()), 1)}

        out = {"workload": wl.name, "straggler_rank": lag, "n0": n0,
               "calibration": {"undelayed_ms": round(ms0, 4), "pieces": plan.work_items,
                               "workgroups": wg, "t_piece_us": round(t_piece_us, 3),
                               "rule": "n0 = t_piece / 1.5 ticks of 10 ns: a delayed piece waits "
                                       "t_piece on average, taking about twice a clean one"},
               "note": "per-tile completion stamps (device clock), microseconds from the launch's "
                       "first stamp; SET per (tile, source): each source's tiles separately"}
        for name, mode in (("direct", 0), ("staged", ra2a.MODE_STAGED)):
            msu, lag_u, oth_u = run(0, mode)
            ms, lagged, others = run(n0, mode)
            out[name] = {
                "ms_delayed": round(ms, 4), "ms_undelayed": round(msu, 4),
                "delayed_source_us": q(lagged), "other_sources_us": q(others),
                "undelayed": {"that_source_us": q(lag_u), "other_sources_us": q(oth_u)},
                "median_lag_us": round(float(np.median(lagged) - np.median(others)), 1),
                # behind a barrier every tile would complete after the last piece of
                # every source; with per-tile signals this share of the other
                # sources' tiles is complete before the delayed source's last tile
                "other_tiles_done_before_delayed_last": round(float((others < lagged.max()).mean()), 4)}
        out["parity"] = combine_views_match(heap, oi, oo, wl, torch.int32)
        return out
    finally:
        heap.close()


def copy_ceiling(nbytes, steps):
    """The practical ceiling for copy-shaped traffic: torch's device copy of one
    contiguous buffer of `nbytes` into another, over NSETS rotated pairs so that,
    as in the timed combine, no step finds its data in the 256 MB MALL."""
    import torch

    pairs = [(torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
              torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(NSETS)]
    st = torch.cuda.current_stream()
    for k in range(2 * NSETS):
        pairs[k % NSETS][1].copy_(pairs[k % NSETS][0])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for k in range(steps):
        pairs[k % NSETS][1].copy_(pairs[k % NSETS][0])
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    del pairs
    return {"what": f"torch copy of {nbytes >> 20} MiB, {NSETS} rotated buffer pairs (cold in the MALL)",
            "ms": round(ms, 5), "GBps": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--legs", choices=["all", "main", "moe", "straggler", "ag_gemm", "gemm_rs",
                                       "alltoallv", "staged_ring"], default="all")
    ap.add_argument("--tile-s", type=int, default=64, help="staged_ring leg: tokens per tile")
    ap.add_argument("--ring", type=int, default=8, help="staged_ring leg: ring depth in S-blocks")
    ap.add_argument("--workload", default=WORKLOAD)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the combine's W ranks are simulated as W slices of one heap on one "
              f"GPU; --gpus {args.gpus} is not supported (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_all2all_combine_amd as ra2a
    import synthgen

    if args.legs == "ag_gemm":  # only the AllGather+GEMM leg (for counter runs)
        torch.cuda.set_device(0)
        print(json.dumps({"ag_gemm": ag_gemm_leg(args.steps)}), flush=True)
        return
    if args.legs == "gemm_rs":  # only the GEMM+ReduceScatter leg (for counter runs)
        torch.cuda.set_device(0)
        print(json.dumps({"gemm_rs": gemm_rs_leg(args.steps)}), flush=True)
        return
    if args.legs == "alltoallv":  # only the variable-size AllToAll leg (for counter runs)
        torch.cuda.set_device(0)
        print(json.dumps({"alltoallv": alltoallv_leg(args.steps)}), flush=True)
        return
    if args.legs == "moe":  # only the MoE-combine-shaped leg's default (for counter runs)
        torch.cuda.set_device(0)
        print(json.dumps({"moe_combine": moe_leg(args.steps, profile=True)}), flush=True)
        return
    if args.legs == "staged_ring":  # the staged mode at one ring size (for counter runs)
        torch.cuda.set_device(0)
        print(json.dumps({"staged_ring": staged_ring_leg(args.steps, args.warmup, args.tile_s, args.ring)}),
              flush=True)
        return
    if args.legs == "straggler":
        torch.cuda.set_device(0)
        print(json.dumps({"straggler": straggler_leg()}), flush=True)
        return

    wl = synthgen.WORKLOADS[args.workload]
    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    torch.cuda.set_device(0)
    proto = ra2a.PROTO_SET if wl.protocol == synthgen.PROTOCOL_SET else ra2a.PROTO_ADD
    tiles = dict(tile_s=wl.tile_s, tile_h=wl.tile_h, tile_d=wl.tile_d, protocol=proto)
    opts_lib = ra2a.Opts(**tiles)  # the library's own reset (in-launch in direct mode)
    opts = ra2a.Opts(skip_reset=1, **tiles)
    opts_st = ra2a.Opts(skip_reset=1, mode=ra2a.MODE_STAGED, **tiles)
    # two-phase layout with per-(S-block, sender) signals (forces the SET layout)
    opts_bk = ra2a.Opts(skip_reset=1, mode=ra2a.MODE_BULK,
                        **{k: v for k, v in tiles.items() if k != "protocol"})
    opts_pl = ra2a.Opts(skip_reset=1, mode=ra2a.MODE_PULL,
                        **{k: v for k, v in tiles.items() if k != "protocol"})
    dopts = ra2a.Opts(direction=ra2a.DIR_DISPATCH, **tiles)  # forward All2All, same buffers
    nsig = max(sum(ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, o))
               for o in (opts, opts_st, opts_bk, opts_pl, dopts))  # each set's signal array holds any
    nsig_c = max(sum(ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, o))
                 for o in (opts, opts_st, opts_bk, opts_pl))  # what a separate reset launch clears
    ring = sum(ra2a.rev_all2all_workspace_bytes(W, S, H, D, wl.dtype, o) for o in (opts_st, opts_bk))
    full = ra2a.rev_all2all_workspace_bytes(W, S, H, D, wl.dtype, None, True)
    nb = wl.bytes_per_rank
    # inputs and outputs on 2 MiB boundaries (the header's placement note)
    slice_bytes = NSETS * (2 * nb + nsig * 128 + 4096 + 2 * BIG_ALIGN) + ring + full + (4 << 20)
    heap = ra2a.SymmHeap(W, slice_bytes)
    sets = [(heap.alloc(nb, BIG_ALIGN), heap.alloc(nb, BIG_ALIGN), heap.alloc(nsig * 128))
            for _ in range(NSETS)]
    log(f"[bench] generating {wl.name}")
    ins = synthgen.make_inputs(wl)
    bits = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[wl.elem_bytes]
    npbits = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}[wl.elem_bytes]
    for (oi, _, _) in sets:
        for r in range(W):
            heap.view(oi, (S * W, H, D), bits, r).copy_(torch.from_numpy(ins[r].view(npbits)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority
    hs = heap.handle
    # Steps rotate over NSETS buffer sets, each with its own signal array, so the
    # reset of step k's signals depends only on the last combine that used the
    # same set (step k - NSETS).  Overlapped steps issue each reset on a side
    # stream, where it runs during the previous step's combine; every step still
    # resets its signals before its combine starts (event order).
    done = [None] * NSETS

    def step(k, o, overlap=True, reset=True, nsets=NSETS):
        oi, oo, osg = sets[k % nsets]
        if not reset:
            pass  # the combine zeroes its own signals
        elif overlap:
            if done[k % NSETS] is not None:
                side.wait_event(done[k % NSETS])
            ra2a.signal_reset(hs, heap.ptr(osg), nsig_c, side)
            ready = torch.cuda.Event()
            ready.record(side)
            stream.wait_event(ready)
        else:
            ra2a.signal_reset(hs, heap.ptr(osg), nsig_c, stream)
        ra2a.rev_all2all_ex(heap.ptr(oi), heap.ptr(oo), heap.ptr(osg), W, S, H, D, wl.dtype, o,
                            stream)
        if overlap and reset:
            fin = torch.cuda.Event()
            fin.record(stream)
            done[k % NSETS] = fin

    def timed(o, steps, warmup, overlap=True, reset=True, nsets=NSETS):
        """Wall-clock ms per step, and ms per step between two HIP events recorded
        on the launch stream around the whole timed region."""
        for k in range(warmup):
            step(k, o, overlap=overlap, reset=reset, nsets=nsets)
        torch.cuda.synchronize()
        assert ra2a.check(hs) == ra2a.OK, ra2a.last_error()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for k in range(steps):
            step(k, o, overlap, reset, nsets)
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        assert ra2a.check(hs) == ra2a.OK, ra2a.last_error()
        return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps

    if args.legs == "main":  # counter runs: a copy of known size in the same process
        put_calibration(heap, sets[0][0], sets[0][1], nb)
    # No timing events between launches (a timestamped event between two kernels
    # costs microseconds per step on this stack).  An in-launch step is exactly
    # one launch of the persistent kernel, so the events around its timed region
    # give the kernel's average launch duration (launch to launch, gaps included).
    log(f"[bench] {args.warmup} warmup + {args.steps} timed steps")
    inl_ms, kern_ms = timed(opts_lib, args.steps, args.warmup, overlap=False, reset=False)
    serial_ms, _ = timed(opts, args.steps, args.warmup, overlap=False)
    overlap_ms, _ = timed(opts, args.steps, args.warmup, overlap=True)
    # warm, for context only: every step on one buffer set, whose 256 MiB the
    # 256 MB MALL largely holds from one step to the next
    warm_ms, warm_kern_ms = timed(opts_lib, args.steps, args.warmup, overlap=False, reset=False, nsets=1)
    variants = {"in_launch": inl_ms, "serial": serial_ms, "overlapped": overlap_ms}
    mode_used = min(variants, key=variants.get)
    ms_per_step = variants[mode_used]

    n_tile = ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, opts)[0]

    def parity(k, check_signals=True):
        """Output of step k satisfies the definition out_j[s, r*H + h, d] =
        in_r[j*S + s, h, d], compared as bits on the device with torch views, and
        (ADD) every tile signal reads W."""
        oi, oo, osg = sets[k % NSETS]
        ok = all(torch.equal(heap.view(oo, (S, W, H, D), bits, j)[:, r],
                             heap.view(oi, (W, S, H, D), bits, r)[j])
                 for j in range(W) for r in range(W))
        if check_signals and wl.protocol != synthgen.PROTOCOL_SET:
            ok = ok and all(bool((heap.view(osg, (n_tile, ra2a.SIG_STRIDE_U64), torch.int64, j)[:, 0]
                                  == W).all()) for j in range(W))
        return ok

    def poison(k):
        """Outputs and signal array of buffer set k filled with garbage."""
        _, oo, osg = sets[k % NSETS]
        for j in range(W):
            heap.view(oo, (nb,), torch.uint8, j).fill_(0xA5)
            heap.view(osg, (nsig * 128,), torch.uint8, j).fill_(0x5A)
        torch.cuda.synchronize()

    # parity of the headline variant itself: set 0 poisoned, one more in-launch step
    poison(0)
    step(0, opts_lib, overlap=False, reset=False)
    torch.cuda.synchronize()
    ok = ra2a.check(hs) == ra2a.OK and parity(0)
    log(f"[bench] combine {ms_per_step * 1e3:.1f} us/step, kernel {kern_ms * 1e3:.1f} us, "
        f"parity {ok}")
    alg = wl.algorithmic_bytes
    value = alg / (ms_per_step * 1e-3) / 1e9
    achieved = alg / (kern_ms * 1e-3) / 1e9
    rec = {
        "metric": "Reverse-All2All combine GB/s (read+write) and % of HBM peak, W=8 bf16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "parity": ok,
        "config": {"workload": wl.name, "W": W, "S": S, "H": H, "D": D, "dtype": wl.dtype,
                   "tile": [wl.tile_s, wl.tile_h, wl.tile_d], "protocol": wl.protocol,
                   "variant": "signal-pipelined persistent kernel, direct mode, " + MODE_NAMES.get(
                       ra2a.rev_all2all_plan(W, S, H, D, wl.dtype, opts_lib).mode, "?"),
                   "step": "signal reset + combine", "steps_issued": mode_used,
                   "buffer_sets": NSETS,
                   "algorithmic_bytes": alg},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(),
                     "kernel": kernel_label(ra2a.rev_all2all_plan(W, S, H, D, wl.dtype, opts_lib).mode),
                     "kernel_ms": round(kern_ms, 5)},
    }
    rec["step_variants"] = {
        "in_launch": {"ms_per_step": round(inl_ms, 5),
                      "note": "one launch per step; its first workgroups zero the signals"},
        "serial": {"ms_per_step": round(serial_ms, 5),
                   "note": "a reset launch and the combine back to back on one stream"},
        "overlapped": {"ms_per_step": round(overlap_ms, 5),
                       "note": "each reset launch on a side stream during the previous step's combine"},
        "kernel_timing": "HIP events on the launch stream around the in-launch timed region / launches"}
    rec["warm"] = {"ms_per_step": round(warm_ms, 5), "value": round(alg / (warm_ms * 1e-3) / 1e9, 2),
                   "kernel_ms": round(warm_kern_ms, 5),
                   "note": "context, not the headline: in-launch steps on one buffer set, data left in "
                           f"the MALL by the previous step; the headline rotates {NSETS} sets (cold)"}
    if args.legs == "all":
        # the other direct mode, in-launch reset as the headline
        opts_pc = ra2a.Opts(mode=ra2a.MODE_DIRECT, **tiles)
        pc_ms, pc_kern_ms = timed(opts_pc, args.steps, args.warmup, overlap=False, reset=False)
        poison(0)
        step(0, opts_pc, overlap=False, reset=False)
        torch.cuda.synchronize()
        rec["pieces"] = {"ms_per_step": round(pc_ms, 5), "kernel_ms": round(pc_kern_ms, 5),
                         "value": round(alg / (pc_ms * 1e-3) / 1e9, 2),
                         "parity": ra2a.check(hs) == ra2a.OK and parity(0),
                         "note": "RA2A_MODE_DIRECT: per-source pieces, in-launch reset"}
        st_ms, _ = timed(opts_st, args.steps, args.warmup, overlap=False)  # reset launch + combine
        poison(0)
        step(0, opts_st, overlap=False)
        torch.cuda.synchronize()
        st_ok = ra2a.check(hs) == ra2a.OK and parity(0)
        rec["staged"] = {"ms_per_step": round(st_ms, 5),
                         "value": round(alg / (st_ms * 1e-3) / 1e9, 2), "parity": st_ok}
        bk_ms, _ = timed(opts_bk, args.steps, args.warmup, overlap=False)  # reset launch + combine
        poison(0)
        step(0, opts_bk, overlap=False)
        torch.cuda.synchronize()
        rec["bulk"] = {"ms_per_step": round(bk_ms, 5),
                       "value": round(alg / (bk_ms * 1e-3) / 1e9, 2),
                       "parity": ra2a.check(hs) == ra2a.OK and parity(0, check_signals=False),
                       "note": "two-phase layout with per-(S-block, sender) signals"}
        pl_ms, _ = timed(opts_pl, args.steps, args.warmup, overlap=False)  # reset launch + combine
        poison(0)
        step(0, opts_pl, overlap=False)
        torch.cuda.synchronize()
        rec["pull"] = {"ms_per_step": round(pl_ms, 5),
                       "value": round(alg / (pl_ms * 1e-3) / 1e9, 2),
                       "parity": ra2a.check(hs) == ra2a.OK and parity(0, check_signals=False),
                       "note": "pull mode: senders stage in their own slice, receivers pull"}

        # forward All2All (dispatch, the combine's inverse) on the same buffers
        # (in_j read as (S, H*W, D), out_r written as (S*W, H, D)), in-launch reset

        def dispatch(k):
            oi, oo, osg = sets[k % NSETS]
            ra2a.all2all_dispatch_ex(heap.ptr(oi), heap.ptr(oo), heap.ptr(osg), W, S, H, D,
                                     wl.dtype, dopts, stream)

        for k in range(args.warmup):
            dispatch(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            dispatch(k)
        torch.cuda.synchronize()
        d_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        assert ra2a.check(hs) == ra2a.OK, ra2a.last_error()
        # the definition out_r[j*S + s, h, d] = in_j[s, r*H + h, d], as bits on the device
        d_oi, d_oo, _ = sets[(args.steps - 1) % NSETS]
        d_ok = all(torch.equal(heap.view(d_oo, (W, S, H, D), bits, r)[j],
                               heap.view(d_oi, (S, W, H, D), bits, j)[:, r])
                   for j in range(W) for r in range(W))
        rec["dispatch"] = {"ms_per_step": round(d_ms, 5),
                           "value": round(alg / (d_ms * 1e-3) / 1e9, 2), "parity": d_ok,
                           "note": "forward All2All (the combine's inverse), one launch per step"}

        def two_phase(k):
            oi, oo, _ = sets[k % NSETS]
            ra2a.rev_all2all_two_phase(heap.ptr(oi), heap.ptr(oo), None, W, S, H, D, wl.dtype,
                                       stream)

        def put_copy(k):
            # calibration copy: every in slice -> the out slot of the same slice
            oi, oo, _ = sets[k % NSETS]
            for r in range(W):
                ra2a.put(hs, heap.ptr(oo), heap.ptr(oi, r), nb, r, stream)

        ctx = {}
        for name, fn in (("two_phase", two_phase), ("put_copy", put_copy)):
            for k in range(args.warmup):
                fn(k)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(args.steps):
                fn(k)
            torch.cuda.synchronize()
            ctx[name] = (time.perf_counter() - t0) * 1e3 / args.steps
        rec["two_phase"] = {"ms_per_step": round(ctx["two_phase"], 5),
                            "value": round(alg / (ctx["two_phase"] * 1e-3) / 1e9, 2)}
        rec["put_copy"] = {"bytes_moved": 2 * W * nb, "launches": W,
                           "ms": round(ctx["put_copy"], 5),
                           "GBps": round(2 * W * nb / (ctx["put_copy"] * 1e-3) / 1e9, 2)}
        rec["copy_ceiling"] = copy_ceiling(W * nb, args.steps)
    heap.close()
    if args.legs == "all":
        log("[bench] MoE-combine-shaped leg")
        rec["moe_combine"] = moe_leg(10)
        log("[bench] straggler leg")
        rec["straggler"] = straggler_leg()
        log("[bench] GEMM legs")
        rec["ag_gemm"] = ag_gemm_leg(args.steps // 5 + 3)
        rec["gemm_rs"] = gemm_rs_leg(args.steps // 5 + 3)
        rec["alltoallv"] = alltoallv_leg(args.steps // 5 + 3)
    rec["cpu_baseline"] = None if args.no_cpu else cpu_baseline(wl, ins)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
