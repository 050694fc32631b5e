#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet recurrent-state hot path on one MI355X.

A step is one decode token for a batch of 512 requests through 48 GDN layers
run back to back (one 512-slot BF16 state pool per layer, in-place slots,
H_qk = 16, H_v = 32, d_k = d_v = 128), each layer one gdn_decode launch.  The
48 launches are captured in one HIP graph and replayed.  Inputs are seeded
synthetic tensors already resident in HBM.

Prints ONE JSON line: tokens/s, state GB/s and the fraction of HBM peak for
the decode kernel, the CPU oracle timed on a bounded sample of the same
workload, and (when built) chunked-prefill tokens/s.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN decode state-update GB/s (% HBM peak) + tokens/s at B=512; prefill tok/s"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0
DECODE_SOURCES = ["csrc/decode.cuh", "csrc/decode.hip", "csrc/device.h", "csrc/order.cuh"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_b512_x48_counters.txt")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def decode_source_hash() -> str:
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "linear_attention_recurrent_02_amd")
    for rel in DECODE_SOURCES:
        with open(os.path.join(pkg, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter runs,
    valid only if the decode sources still hash to what was profiled."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    for line in open(COUNTERS_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.get("source_hash") != decode_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def decode_bytes_per_launch(B, H_qk, H_v, d_k, d_v, state_bytes=2, act_bytes=2):
    """Algorithmic bytes of one decode launch: each state tile read once and
    written once, q, k, v read, o written, g and beta read."""
    state = 2 * B * H_v * d_k * d_v * state_bytes
    acts = B * (2 * H_qk * d_k + 2 * H_v * d_v) * act_bytes
    gates = 2 * B * H_v * 4
    return state, acts + gates


def run_decode(args, torch, gdn, syn):
    wl = syn.WORKLOADS["decode_b512_x48"]
    B, Hqk, Hv, dk, dv, n = wl["B"], wl["H_qk"], wl["H_v"], wl["d_k"], wl["d_v"], wl["n_slots"]
    L = args.layers
    log(f"decode setup: B={B} H_qk={Hqk} H_v={Hv} d={dk} layers={L} (pools {L * n} MiB)")
    t0 = time.time()
    layers = []
    for l in range(L):
        q, k, v, g, beta = (t.cuda() for t in syn.token_inputs(wl["index"], l, B, Hqk, Hv, dk, dv))
        pool = syn.state_pool(wl["index"], l, n, Hv, dk, dv, torch.bfloat16, on_device=True)
        rs, ws = (t.cuda() for t in syn.distinct_slots(wl["index"], l, n, B, in_place=True))
        a, o, keep = gdn.make_decode_args(q, k, v, g, beta, pool, rs, ws)
        layers.append((a, keep))
    torch.cuda.synchronize()
    log(f"decode setup done in {time.time() - t0:.1f}s")
    lib = gdn.load_library()

    def step():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for a, _ in layers:
            code = lib.gdn_decode(ctypes.byref(a), s)
            if code:
                raise gdn.GdnError("gdn_decode", code)

    run = step
    if not args.no_graph:
        step()  # load the code object before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    state_b, other_b = decode_bytes_per_launch(B, Hqk, Hv, dk, dv)
    per_launch = state_b + other_b
    launch_s = ms_step / 1e3 / L
    res = dict(B=B, H_qk=Hqk, H_v=Hv, d=dk, layers=L, ms_per_step=ms_step,
               tokens_per_s=B / (ms_step / 1e3),
               state_GBps=L * state_b / (ms_step / 1e3) / 1e9,
               total_GBps=L * per_launch / (ms_step / 1e3) / 1e9,
               avg_launch_us=launch_s * 1e6, bytes_per_launch=per_launch)
    return res, layers


def run_cpu_baseline(args, torch, layers, syn):
    """The FP64 oracle on layers 0 and L-1 at full batch (every request-head),
    timed on this host's cores; tokens/s extrapolated to all layers."""
    import numpy as np
    import oracle

    threads = len(os.sched_getaffinity(0))
    times = []
    picks = sorted({0, len(layers) - 1})
    for l in picks:
        _, keep = layers[l]
        q, k, v, g, beta, pool, rs, ws = keep[:8]
        f = lambda t: t.detach().to("cpu", torch.float64).numpy()
        hq, hk, hv, hg, hb = f(q), f(k), f(v), f(g), f(beta)
        hpool = f(pool)
        hrs, hws = rs.cpu().numpy(), ws.cpu().numpy()
        t0 = time.perf_counter()
        oracle.decode(hq, hk, hv, hg, hb, hpool, hrs, hws, round_state=True, n_threads=threads)
        times.append(time.perf_counter() - t0)
        del hpool
    B = layers[0][1][0].shape[0]
    per_layer = sum(times) / len(times)
    return dict(value=B / (per_layer * len(layers)), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"FP64 oracle on layers {picks} of {len(layers)} at B={B} (all request-heads), "
                       f"{per_layer:.2f}s per layer; tokens/s extrapolated to {len(layers)} layers")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a device copy of known size (for counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_recurrent_02_amd as gdn
    from linear_attention_recurrent_02_amd import synthetic as syn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gdn.load_library()
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.total_memory / 2**30:.0f} GiB")

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {n} bytes")
        del src, dst

    dec, layers = run_decode(args, torch, gdn, syn)
    achieved = dec["bytes_per_launch"] / (dec["avg_launch_us"] / 1e6) / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=recorded_traffic(),
                    kernel="decode_kernel<bf16 state, bf16 act, 128, 128>",
                    per_launch_bytes=dec["bytes_per_launch"],
                    avg_launch_us=round(dec["avg_launch_us"], 2))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(args, torch, layers, syn)
    out = {
        "metric": METRIC,
        "value": round(dec["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode_b512_x48", "B": dec["B"], "layers": dec["layers"],
                   "H_qk": dec["H_qk"], "H_v": dec["H_v"], "d_k": dec["d"], "d_v": dec["d"],
                   "state_storage": "bf16", "activations": "bf16", "rule": "gated_delta",
                   "slots": "in place, seeded permutation", "hip_graph": not args.no_graph},
        "state_GBps": round(dec["state_GBps"], 1),
        "total_GBps": round(dec["total_GBps"], 1),
        "hbm_frac": round(dec["total_GBps"] / HBM_PEAK_GBPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
