"""Benchmark of the Reverse All2All combine on one MI355X.

One step = one whole combine (signal reset + the signal-pipelined persistent
kernel) over the EP-combine workload: W=8 simulated ranks, S=512 tokens, H=16
heads, D=128, bf16 values uniform(-1, 1) from seed 0, 64 x 1 x 128 tiles with
ADD-to-W tile signals.  Inputs are resident in HBM before timing starts.  To
keep the 256 MiB working set from being served by the 256 MB Infinity Cache,
consecutive steps rotate through several independent in/out buffer sets.

Prints one JSON line (metric, value in GB/s of algorithmic bytes = every input
element read once + every output element written once, roofline of the
persistent kernel from HIP events around its launches, the two-phase variant
and a plain device copy for context, and the CPU oracle's rate on the host).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "ep_combine_w8_s512_h16_d128_bf16"
HBM_PEAK_GBS = 8000.0
NSETS = 6


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(wl, budget_s=12.0):
    """The CPU oracle (single thread) on repeated full combines for about budget_s."""
    import oracle
    import synthgen

    ins = synthgen.make_inputs(wl)
    oracle.combine(ins)  # warm
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.combine(ins)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    gbs = wl.algorithmic_bytes * reps / el / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full combines of the {wl.name} workload, single thread, "
                      f"{el:.1f} s"}


def load_traffic():
    """HBM traffic of the persistent kernel from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_rev_a2a_pipelined_ep_combine_w8.json")
    if not os.path.exists(path):
        return None
    import hashlib
    src = os.path.join(ROOT, "moe_all2all_combine_amd", "csrc", "combine_kernels.hip")
    dev = os.path.join(ROOT, "moe_all2all_combine_amd", "csrc", "device.h")
    h = hashlib.sha256(open(src, "rb").read() + open(dev, "rb").read()).hexdigest()[:16]
    rec = json.load(open(path))
    if rec.get("source_hash") != h:
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--workload", default=WORKLOAD)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs the combine's W simulated ranks on one GPU; "
              f"--gpus {args.gpus} is not supported (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_all2all_combine_amd as ra2a
    import synthgen

    wl = synthgen.WORKLOADS[args.workload]
    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    torch.cuda.set_device(0)
    proto = ra2a.PROTO_SET if wl.protocol == synthgen.PROTOCOL_SET else ra2a.PROTO_ADD
    opts = ra2a.Opts(tile_s=wl.tile_s, tile_h=wl.tile_h, tile_d=wl.tile_d, protocol=proto)
    opts_nr = ra2a.Opts(tile_s=wl.tile_s, tile_h=wl.tile_h, tile_d=wl.tile_d, protocol=proto,
                        skip_reset=1)
    n_tile, n_credit = ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, opts)
    nsig = n_tile + n_credit
    ring = ra2a.rev_all2all_workspace_bytes(W, S, H, D, wl.dtype, opts)
    full = ra2a.rev_all2all_workspace_bytes(W, S, H, D, wl.dtype, None, True)
    nb = wl.bytes_per_rank
    slice_bytes = NSETS * (2 * nb + nsig * 128 + 4096) + ring + full + (1 << 20)
    heap = ra2a.SymmHeap(W, slice_bytes)
    sets = []
    for _ in range(NSETS):
        sets.append((heap.alloc(nb), heap.alloc(nb), heap.alloc(nsig * 128)))
    log(f"[bench] generating {wl.name}")
    ins = synthgen.make_inputs(wl)
    bits = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[wl.elem_bytes]
    for (oi, _, _) in sets:
        for r in range(W):
            heap.view(oi, (S * W, H, D), bits, r).copy_(
                torch.from_numpy(ins[r].view({2: np.int16, 4: np.int32, 1: np.uint8,
                                              8: np.int64}[wl.elem_bytes])))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    hs = heap.handle

    def step(k, ev=None):
        oi, oo, osg = sets[k % NSETS]
        ra2a.signal_reset(hs, heap.ptr(osg), nsig, stream)
        if ev is not None:
            ev[0].record(stream)
        ra2a.rev_all2all_ex(heap.ptr(oi), heap.ptr(oo), heap.ptr(osg), W, S, H, D, wl.dtype,
                            opts_nr, stream)
        if ev is not None:
            ev[1].record(stream)

    log("[bench] warmup")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    assert ra2a.check(hs) == ra2a.OK, ra2a.last_error()

    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert ra2a.check(hs) == ra2a.OK, ra2a.last_error()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # kernel-only durations (HIP events on the launch stream, around the persistent kernel)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for k in range(args.steps):
        step(k, evs[k])
    torch.cuda.synchronize()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # parity spot check of the last set used against the oracle (full, W outputs)
    import oracle
    want = oracle.combine(ins)
    oo = sets[(args.steps - 1) % NSETS][1]
    parity = all(heap.view(oo, (S, H * W, D), bits, j).cpu().numpy().tobytes() == want[j].tobytes()
                 for j in range(W))

    # two-phase variant on the same rotation, for context
    for k in range(args.warmup):
        oi, oo, _ = sets[k % NSETS]
        ra2a.rev_all2all_two_phase(heap.ptr(oi), heap.ptr(oo), None, W, S, H, D, wl.dtype, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        oi, oo, _ = sets[k % NSETS]
        ra2a.rev_all2all_two_phase(heap.ptr(oi), heap.ptr(oo), None, W, S, H, D, wl.dtype, stream)
    torch.cuda.synchronize()
    tp_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # a plain device-to-device copy of the same bytes (torch), for context
    src = torch.empty(W * nb, dtype=torch.uint8, device="cuda")
    dsts = [torch.empty_like(src) for _ in range(3)]
    for k in range(3):
        dsts[k].copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        dsts[k % 3].copy_(src)
    torch.cuda.synchronize()
    copy_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    alg = wl.algorithmic_bytes
    value = alg / (ms_per_step * 1e-3) / 1e9
    achieved = alg / (kern_ms * 1e-3) / 1e9
    cpu = None if args.no_cpu else cpu_baseline(wl)
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
        "parity": parity,
        "config": {"workload": wl.name, "W": W, "S": S, "H": H, "D": D, "dtype": wl.dtype,
                   "tile": [wl.tile_s, wl.tile_h, wl.tile_d], "protocol": wl.protocol,
                   "variant": "signal-pipelined persistent kernel", "buffer_sets": NSETS,
                   "algorithmic_bytes": alg},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(), "kernel": "rev_a2a_pipelined_kernel",
                     "kernel_ms": round(kern_ms, 5)},
        "two_phase": {"ms_per_step": round(tp_ms, 5),
                      "value": round(alg / (tp_ms * 1e-3) / 1e9, 2)},
        "device_copy": {"bytes": 2 * W * nb, "ms": round(copy_ms, 5),
                        "GBps": round(2 * W * nb / (copy_ms * 1e-3) / 1e9, 2)},
        "cpu_baseline": cpu,
    }
    heap.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
