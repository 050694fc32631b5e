#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet recurrent-state hot path on one MI355X.

A step is one decode token for a batch of 512 requests through 48 GDN layers
run back to back (one 512-slot BF16 state pool per layer, in-place slots,
H_qk = 16, H_v = 32, d_k = d_v = 128), each layer one gdn_decode launch.  The
48 launches are captured in one HIP graph and replayed.  Inputs are seeded
synthetic tensors already resident in HBM.

Prints ONE JSON line: tokens/s, state GB/s and the fraction of HBM peak for
the decode kernel, the CPU oracle timed on a bounded sample of the same
workload, the decode-side conv front-end (alone and ahead of each layer's
decode), the decode with a per-key-channel decay, chunked-prefill tokens/s
and the mixed launch.
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


def run_copy(args, torch):
    """A plain device-to-device copy of 1 GiB (torch's copy kernel), timed
    like the decode: the practical streaming ceiling on this machine."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return dict(bytes_moved=2 * n, ms=round(ms, 4), GBps=round(2 * n / (ms / 1e3) / 1e9, 1))


def run_decode_b64(args, torch, gdn, syn):
    """The B = 64 decode step (H_qk = 16, H_v = 32, d = 128, 64 live slots of a
    256-slot BF16 pool, distinct read and write slots) for each update rule.
    Its 134 MB of state would sit in the 256 MB last-level cache if one pool
    were reused, so each timed step runs the call once on each of 8
    independent pools (2 GiB in all) in turn; one HIP graph per rule."""
    wl = syn.WORKLOADS["decode_b64"]
    B, Hqk, Hv, dk, dv, n = wl["B"], wl["H_qk"], wl["H_v"], wl["d_k"], wl["d_v"], wl["n_slots"]
    P = 8
    pools = []
    for p in range(P):
        q, k, v, g, beta = (t.cuda() for t in syn.token_inputs(wl["index"], p, B, Hqk, Hv, dk, dv))
        pool = syn.state_pool(wl["index"], p, n, Hv, dk, dv, torch.bfloat16, on_device=True)
        rs, ws = (t.cuda() for t in syn.distinct_slots(wl["index"], p, n, B, in_place=False))
        pools.append((q, k, v, g, beta, pool, rs, ws))
    torch.cuda.synchronize()
    lib = gdn.load_library()
    state_b, other_b = decode_bytes_per_launch(B, Hqk, Hv, dk, dv)
    per_launch = state_b + other_b
    out = {}
    for rule in ("linear", "gated", "delta", "gated_delta"):
        calls = [gdn.make_decode_args(*t[:8], rule=rule) for t in pools]

        def step():
            s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for a, _, _ in calls:
                code = lib.gdn_decode(ctypes.byref(a), s)
                if code:
                    raise gdn.GdnError("gdn_decode", code)

        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 4 * args.steps
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * P)
        gbps = per_launch / (us / 1e6) / 1e9
        out[rule] = dict(avg_launch_us=round(us, 2), algorithmic_GBps=round(gbps, 1),
                         hbm_frac=round(gbps / HBM_PEAK_GBPS, 4),
                         tokens_per_s=round(B / (us / 1e6), 1))
    return dict(workload="decode_b64 (64 of 256 slots, distinct read/write, 8 rotating pools)",
                kernel="decode_kernel<bf16 state, bf16 act, 128, 128>", per_launch_bytes=per_launch,
                pools=P, rules=out)


def conv_bytes_per_launch(B, H_qk, H_v, d_k, d_v, act_bytes=2):
    """Algorithmic bytes of one conv-decode launch: per request the raw row in,
    the q|k|v row out, the 3-token window read and written; a/b in, g/beta
    out; the conv taps (FP32, 4 per channel) once."""
    C = 2 * H_qk * d_k + H_v * d_v
    return B * C * act_bytes * (1 + 1 + 3 + 3) + B * H_v * 4 * 4 + C * 4 * 4


def fused_bytes_per_launch(B, H_qk, H_v, d_k, d_v, act_bytes=2, state_bytes=2):
    """Algorithmic bytes of one fused conv + decode launch: per (request, state
    head) the state tile read and written and o written; per request the raw
    q|k|v row in, the 3-token conv window read and written, a and b in; the
    taps (FP32, 4 per channel) once."""
    C = 2 * H_qk * d_k + H_v * d_v
    state = 2 * B * H_v * d_k * d_v * state_bytes
    return (state + B * H_v * d_v * act_bytes + B * C * act_bytes * (1 + 3 + 3)
            + B * H_v * 2 * 4 + C * 4 * 4)


def run_conv(args, torch, gdn, syn, layers):
    """The decode-side front-end for the same 48-layer B=512 batch: one
    gdn_conv_decode launch per layer (a 512-slot BF16 conv pool per layer, the
    layer's state slots), writing the q, k, v, g, beta that the layer's
    gdn_decode reads.  Times the conv launches alone and the full decode step
    (conv then decode, per layer), each captured in one HIP graph."""
    wl = syn.WORKLOADS["decode_b512_x48"]
    B, Hqk, Hv, dk, dv, n = wl["B"], wl["H_qk"], wl["H_v"], wl["d_k"], wl["d_v"], wl["n_slots"]
    C = 2 * Hqk * dk + Hv * dv
    convs = []
    for l, (da, keep) in enumerate(layers):
        q, k, v, g, beta, pool, rs, ws = keep[:8]
        x = {kk: vv.cuda() for kk, vv in syn.frontend_inputs(wl["index"], 100 + l, B, Hqk, Hv,
                                                             dk, dv, 4).items()}
        cpool = syn.conv_pool(wl["index"], l, n, C, 4, torch.bfloat16, on_device=True)
        ca, ckeep = gdn.make_conv_args(x["q_raw"], x["k_raw"], x["v_raw"], cpool, H_qk=Hqk,
                                       H_v=Hv, read_slot=rs, write_slot=ws, a_raw=x["a_raw"],
                                       b_raw=x["b_raw"], conv_wq=x["conv_wq"],
                                       conv_wk=x["conv_wk"], conv_wv=x["conv_wv"],
                                       outputs=(q, k, v, g, beta))
        convs.append((ca, ckeep, da))
    torch.cuda.synchronize()
    lib = gdn.load_library()

    def conv_only():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for ca, _, _ in convs:
            code = lib.gdn_conv_decode(ctypes.byref(ca), s)
            if code:
                raise gdn.GdnError("gdn_conv_decode", code)

    def conv_then_decode():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for ca, _, da in convs:
            code = lib.gdn_conv_decode(ctypes.byref(ca), s) or lib.gdn_decode(ctypes.byref(da), s)
            if code:
                raise gdn.GdnError("conv + decode", code)

    # the same layers through the fused call: the decode's token inputs and
    # the conv step's outputs left NULL
    fused = []
    for ca, _, da in convs:
        fd = gdn.DecodeArgs.from_buffer_copy(da)
        fd.q = fd.k = fd.v = fd.g = fd.beta = None
        fc = gdn.ConvArgs.from_buffer_copy(ca)
        fc.q_out = fc.k_out = fc.v_out = fc.g_out = fc.beta_out = None
        fused.append((fd, fc))

    def fused_step():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for fd, fc in fused:
            code = lib.gdn_decode_conv(ctypes.byref(fd), ctypes.byref(fc), s)
            if code:
                raise gdn.GdnError("gdn_decode_conv", code)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        run = fn
        if not args.no_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            torch.cuda.synchronize()
            run = graph.replay
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_conv = timed(conv_only)
    ms_step = timed(conv_then_decode)
    ms_fused = timed(fused_step)
    L = len(convs)
    per_launch = conv_bytes_per_launch(B, Hqk, Hv, dk, dv)
    us = ms_conv * 1e3 / L
    gbps = per_launch / (us / 1e6) / 1e9
    f_bytes = fused_bytes_per_launch(B, Hqk, Hv, dk, dv)
    f_us = ms_fused * 1e3 / L
    f_gbps = f_bytes / (f_us / 1e6) / 1e9
    return dict(workload="decode_b512_x48 front-end", kernel="conv_decode_kernel<bf16, 128>",
                avg_launch_us=round(us, 2), per_launch_bytes=per_launch,
                algorithmic_GBps=round(gbps, 1), hbm_frac=round(gbps / HBM_PEAK_GBPS, 4),
                decode_with_conv_ms_per_step=round(ms_step, 4),
                decode_with_conv_tokens_per_s=round(B / (ms_step / 1e3), 1),
                fused=dict(kernel="decode_conv_bf16_kernel<128, 128>",
                           ms_per_step=round(ms_fused, 4),
                           tokens_per_s=round(B / (ms_fused / 1e3), 1),
                           avg_launch_us=round(f_us, 2), per_launch_bytes=f_bytes,
                           algorithmic_GBps=round(f_gbps, 1),
                           hbm_frac=round(f_gbps / HBM_PEAK_GBPS, 4),
                           vs_separate=round(ms_step / ms_fused, 4)))


def run_conv_small(args, torch, gdn, syn, B=16):
    """The conv + decode step at a small batch (B = 16 requests, the decode
    workload's heads, 48 layers with a B-slot state and conv pool each,
    in-place slots in a seeded permutation): the separate calls against the
    fused gdn_decode_conv, each layer sequence captured in one HIP graph.  At
    this size every launch is short, so the saved launch is what counts."""
    wl = syn.WORKLOADS["decode_b512_x48"]
    Hqk, Hv, d = wl["H_qk"], wl["H_v"], wl["d_k"]
    lib = gdn.load_library()
    sep, fus, keep = [], [], []
    for l in range(args.layers):
        x = {kk: vv.cuda() for kk, vv in syn.frontend_inputs(wl["index"], 200 + l, B, Hqk, Hv, d,
                                                             d, 4).items()}
        pool = syn.state_pool(wl["index"], 200 + l, B, Hv, d, d, torch.bfloat16, on_device=True)
        cpool = syn.conv_pool(wl["index"], 200 + l, B, 2 * Hqk * d + Hv * d, 4, torch.bfloat16,
                              on_device=True)
        slots = syn.distinct_slots(wl["index"], 200 + l, B, B, True)[0].cuda()
        q = torch.empty((B, Hqk, d), dtype=torch.bfloat16, device="cuda")
        k = torch.empty_like(q)
        v = torch.empty((B, Hv, d), dtype=torch.bfloat16, device="cuda")
        g = torch.empty((B, Hv), dtype=torch.float32, device="cuda")
        b = torch.empty_like(g)
        ca, ck = gdn.make_conv_args(x["q_raw"], x["k_raw"], x["v_raw"], cpool, H_qk=Hqk, H_v=Hv,
                                    read_slot=slots, write_slot=slots, a_raw=x["a_raw"],
                                    b_raw=x["b_raw"], conv_wq=x["conv_wq"], conv_wk=x["conv_wk"],
                                    conv_wv=x["conv_wv"], outputs=(q, k, v, g, b))
        da, _, dk = gdn.make_decode_args(q, k, v, g, b, pool, slots, slots)
        fd = gdn.DecodeArgs.from_buffer_copy(da)
        fd.q = fd.k = fd.v = fd.g = fd.beta = None
        fc = gdn.ConvArgs.from_buffer_copy(ca)
        fc.q_out = fc.k_out = fc.v_out = fc.g_out = fc.beta_out = None
        sep.append((ca, da))
        fus.append((fd, fc))
        keep.append((x, pool, cpool, slots, ck, dk))

    def separate():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for ca, da in sep:
            code = lib.gdn_conv_decode(ctypes.byref(ca), s) or lib.gdn_decode(ctypes.byref(da), s)
            if code:
                raise gdn.GdnError("conv + decode", code)

    def fused():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for fd, fc in fus:
            code = lib.gdn_decode_conv(ctypes.byref(fd), ctypes.byref(fc), s)
            if code:
                raise gdn.GdnError("gdn_decode_conv", code)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_sep, ms_fused = timed(separate), timed(fused)
    return dict(workload=f"decode_b{B}_x{len(sep)} with the conv step", B=B,
                separate_ms_per_step=round(ms_sep, 4), fused_ms_per_step=round(ms_fused, 4),
                fused_tokens_per_s=round(B / (ms_fused / 1e3), 1),
                fused_vs_separate=round(ms_sep / ms_fused, 4))


def run_decode_cw(args, torch, gdn, syn, layers):
    """The same 48-layer B=512 decode with a per-key-channel decay (g of shape
    [B, H_v, d_k], Kimi Delta Attention's channel-wise gate): the decode
    kernel's channel-wise instance, one HIP graph of 48 launches."""
    wl = syn.WORKLOADS["decode_b512_x48"]
    B, Hqk, Hv, dk, dv = wl["B"], wl["H_qk"], wl["H_v"], wl["d_k"], wl["d_v"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    cws = []
    for a, keep in layers:
        q, k, v, g, beta, pool, rs, ws = keep[:8]
        gcw = -torch.nn.functional.softplus(
            torch.randn((B, Hv, dk), generator=gen, device="cuda", dtype=torch.float32))
        ca, _, ckeep = gdn.make_decode_args(q, k, v, gcw, beta, pool, rs, ws)
        cws.append((ca, ckeep))
    torch.cuda.synchronize()
    lib = gdn.load_library()

    def step():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for ca, _ in cws:
            code = lib.gdn_decode(ctypes.byref(ca), s)
            if code:
                raise gdn.GdnError("gdn_decode", code)

    step()
    torch.cuda.synchronize()
    run = step
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    state_b, other_b = decode_bytes_per_launch(B, Hqk, Hv, dk, dv)
    per_launch = state_b + other_b + B * Hv * (dk - 1) * 4   # g grows from [B, H_v] to [B, H_v, d_k]
    us = ms * 1e3 / len(cws)
    gbps = per_launch / (us / 1e6) / 1e9
    return dict(workload="decode_b512_x48, per-key-channel decay",
                kernel="decode_kernel<bf16 state, bf16 act, 128, 128, channel decay>",
                ms_per_step=round(ms, 4), tokens_per_s=round(B / (ms / 1e3), 1),
                avg_launch_us=round(us, 2), per_launch_bytes=per_launch,
                algorithmic_GBps=round(gbps, 1), hbm_frac=round(gbps / HBM_PEAK_GBPS, 4))


def run_decode_q8(args, torch, gdn, syn, layers, n_hi=32):
    """The same 48-layer B=512 decode on state pools in the 8-bit format (the
    first n_hi key channels of each tile in BF16, the others INT8 with a
    scale per channel: 10.19 bits per value at n_hi = 32, d = 128; 8.25 with
    none), one HIP graph of 48 launches on 48 separate 8-bit pools."""
    wl = syn.WORKLOADS["decode_b512_x48"]
    B, Hqk, Hv, dk, dv, n = wl["B"], wl["H_qk"], wl["H_v"], wl["d_k"], wl["d_v"], wl["n_slots"]
    calls = []
    for l, (a, keep) in enumerate(layers):
        q, k, v, g, beta, pool, rs, ws = keep[:8]
        qpool = syn.state_pool_q8_bytes(wl["index"], l, n, Hv, dk, dv, n_hi)
        qa, _, qkeep = gdn.make_decode_args(q, k, v, g, beta, qpool, rs, ws, state_bf16_rows=n_hi)
        calls.append((qa, qkeep))
    torch.cuda.synchronize()
    lib = gdn.load_library()

    def step():
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for qa, _ in calls:
            code = lib.gdn_decode(ctypes.byref(qa), s)
            if code:
                raise gdn.GdnError("gdn_decode", code)

    step()
    torch.cuda.synchronize()
    run = step
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    slot = gdn.gdn_state_q8_bytes(Hv, dk, dv, n_hi)
    # algorithmic: the rows, codes and scales each tile holds (not its padding)
    used = Hv * (n_hi * dv * 2 + (dk - n_hi) * (dv + 4))
    state_b = 2 * B * used
    _, other_b = decode_bytes_per_launch(B, Hqk, Hv, dk, dv)
    per_launch = state_b + other_b
    us = ms * 1e3 / len(calls)
    gbps = per_launch / (us / 1e6) / 1e9
    del calls
    return dict(workload="decode_b512_x48, 8-bit state", n_hi=n_hi,
                bits_per_value=round(8 * used / (Hv * dk * dv), 3),
                stored_bits_per_value=round(8 * slot / (Hv * dk * dv), 3),
                state_bytes_vs_bf16=round(slot / (Hv * dk * dv * 2), 4),
                kernel="decode_kernel<q8 state, bf16 act, 128, 128>",
                ms_per_step=round(ms, 4), tokens_per_s=round(B / (ms / 1e3), 1),
                avg_launch_us=round(us, 2), per_launch_bytes=per_launch,
                algorithmic_GBps=round(gbps, 1), hbm_frac=round(gbps / HBM_PEAK_GBPS, 4))


def run_convert(args, torch, gdn, syn, layers, n_hi=32):
    """gdn_state_convert on the decode workload's shape: the 512 BF16 slots of
    a layer's pool stored into an 8-bit pool (n_hi BF16 rows of 128), and back
    into BF16; each direction 20 calls timed with HIP events after 3."""
    wl = syn.WORKLOADS["decode_b512_x48"]
    Hv, dk, dv, n = wl["H_v"], wl["d_k"], wl["d_v"], wl["n_slots"]
    src = layers[0][1][5]
    q8 = torch.zeros((n, Hv, gdn.gdn_state_q8_bytes(1, dk, dv, n_hi)), dtype=torch.uint8,
                     device="cuda")
    b16 = torch.empty_like(src)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 20 * 1e3

    us_in = timed(lambda: gdn.gdn_state_convert(src, q8, dst_bf16_rows=n_hi))
    us_out = timed(lambda: gdn.gdn_state_convert(q8, b16, src_bf16_rows=n_hi))
    bf16_b = n * Hv * dk * dv * 2
    q8_b = n * Hv * (n_hi * dv * 2 + (dk - n_hi) * (dv + 4))
    gb = lambda b, us: round(b / (us / 1e6) / 1e9, 1)
    return dict(workload=f"{n} slots x {Hv} heads of {dk}x{dv}", n_hi=n_hi,
                to_q8_us=round(us_in, 2), to_q8_GBps=gb(bf16_b + q8_b, us_in),
                from_q8_us=round(us_out, 2), from_q8_GBps=gb(bf16_b + q8_b, us_out),
                bytes_moved=bf16_b + q8_b)


def prefill_useful_flops(lengths, H_v, d_k, d_v, C=64):
    """Useful flops of the chunked recurrence (per chunk of n tokens and head):
    K K^T and Q K^T (lower triangle incl. diagonal), the triangular solve,
    U = T R, K M, Q M, (L o Q K^T) U and K~^T U."""
    total = 0
    for T in lengths:
        full, tail = divmod(int(T), C)
        for n in [C] * full + ([tail] if tail else []):
            tri = n * (n + 1) // 2
            f = 2 * tri * d_k * 2            # K K^T, Q K^T
            f += n * n * n // 3              # (I + A)^-1, forward substitution
            f += 2 * tri * d_v               # U = T R (T lower triangular)
            f += 2 * 2 * n * d_k * d_v       # K M, Q M
            f += 2 * tri * d_v               # (L o Q K^T) U
            f += 2 * n * d_k * d_v           # K~^T U
            total += f
    return total * H_v


def run_prefill(args, torch, gdn, syn):
    """Chunked prefill of 8 ragged sequences (1024..8192 tokens, seeded) with
    the fused front-end, H_qk=16, H_v=32, d=128, BF16, fresh requests whose
    final states go to 8 checkpoint slots of a 64-slot pool."""
    import numpy as np
    wl = syn.WORKLOADS["prefill_varlen"]
    Hqk, Hv, d = wl["H_qk"], wl["H_v"], wl["d_k"]
    lengths = syn.seq_lengths(wl["index"], 0, wl["n_seq"], wl["min_len"], wl["max_len"])
    cu = syn.cu_from_lengths(lengths).cuda()
    N = int(lengths.sum())
    x = {k: v.cuda() for k, v in syn.frontend_inputs(wl["index"], 0, N, Hqk, Hv, d, d, 4).items()}
    pool = torch.zeros((wl["n_slots"], Hv, d, d), dtype=torch.bfloat16, device="cuda")
    rs = torch.full((len(lengths),), -1, dtype=torch.int32, device="cuda")
    ws = torch.from_numpy(np.random.default_rng(3).permutation(wl["n_slots"])[:len(lengths)]
                          .astype(np.int32)).cuda()
    a, o, keep = gdn.make_prefill_args(cu, x["q_raw"], x["k_raw"], x["v_raw"], pool, rs, ws,
                                       H_qk=Hqk, H_v=Hv, a_raw=x["a_raw"], b_raw=x["b_raw"],
                                       conv_wq=x["conv_wq"], conv_wk=x["conv_wk"],
                                       conv_wv=x["conv_wv"])
    lib = gdn.load_library()
    s = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        code = lib.gdn_prefill(ctypes.byref(a), s())
        if code:
            raise gdn.GdnError("gdn_prefill", code)

    def fe_only():
        gdn.gdn_frontend(cu, x["q_raw"], x["k_raw"], x["v_raw"], H_qk=Hqk, H_v=Hv,
                         conv_wq=x["conv_wq"], conv_wk=x["conv_wk"], conv_wv=x["conv_wv"],
                         a_raw=x["a_raw"], b_raw=x["b_raw"])

    def timed(fn, reps):
        for _ in range(args.prefill_warmup):  # untimed: the first calls run slower
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(step, args.prefill_reps)
    ms_fe = timed(fe_only, args.prefill_reps)

    # the same call storing an intermediate checkpoint every 1024 tokens (block-aligned prefix
    # cache slots): the pool's slots that are not write slots, 7 per sequence
    ck_every = 1024
    per_seq = int((max(lengths) // ck_every))
    free = np.setdiff1d(np.arange(wl["n_slots"]), ws.cpu().numpy())[:len(lengths) * per_seq]
    ck = torch.from_numpy(free.astype(np.int32).reshape(len(lengths), per_seq)).cuda()
    a_ck, o_ck, keep_ck = gdn.make_prefill_args(cu, x["q_raw"], x["k_raw"], x["v_raw"], pool, rs, ws,
                                                H_qk=Hqk, H_v=Hv, a_raw=x["a_raw"], b_raw=x["b_raw"],
                                                conv_wq=x["conv_wq"], conv_wk=x["conv_wk"],
                                                conv_wv=x["conv_wv"], ckpt_interval=ck_every,
                                                ckpt_slot=ck)

    def step_ck():
        code = lib.gdn_prefill(ctypes.byref(a_ck), s())
        if code:
            raise gdn.GdnError("gdn_prefill", code)

    ms_ck = timed(step_ck, args.prefill_reps)
    n_ck = int(sum(int(L) // ck_every for L in lengths))
    flops = prefill_useful_flops(lengths, Hv, d, d)
    algo_bytes = N * ((2 * Hqk * d + Hv * d) * 2 + Hv * d * 2 + 2 * Hv * 4) + len(lengths) * Hv * d * d * 2
    return dict(workload="prefill_varlen", tokens=N, lengths=[int(v) for v in lengths],
                ms=round(ms, 3), tokens_per_s=round(N / (ms / 1e3), 1),
                frontend_ms=round(ms_fe, 3),
                useful_tflops=round(flops / (ms / 1e3) / 1e12, 2),
                mfma_frac=round(flops / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                algorithmic_GBps=round(algo_bytes / (ms / 1e3) / 1e9, 1),
                hbm_frac=round(algo_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                longest_chain_chunks=int((max(lengths) + 63) // 64),
                ckpt_every_1024_ms=round(ms_ck, 3), ckpt_count=n_ck)


def run_prefill_cw(args, torch, gdn, syn):
    """The chunked-prefill workload's sequences and shapes (8 ragged sequences,
    H_qk=16, H_v=32, d=128, BF16, fresh requests into 8 slots of a 64-slot
    pool) with one decay per key channel (g [N, H_v, d_k] float32, Kimi Delta
    Attention's gate), gated_delta, from final q, k, v, g, beta; beside it the
    scalar-gate chain on the same q, k, v, beta (no front-end in either)."""
    import numpy as np
    wl = syn.WORKLOADS["prefill_varlen"]
    Hqk, Hv, d = wl["H_qk"], wl["H_v"], wl["d_k"]
    lengths = syn.seq_lengths(wl["index"], 0, wl["n_seq"], wl["min_len"], wl["max_len"])
    cu = syn.cu_from_lengths(lengths).cuda()
    N = int(lengths.sum())
    q, k, v, g, beta = syn.token_inputs(wl["index"], 0, N, Hqk, Hv, d, d, on_device=True)
    gcw = syn.channel_gates(wl["index"], 0, N, Hv, d, on_device=True)
    pool = torch.zeros((wl["n_slots"], Hv, d, d), dtype=torch.bfloat16, device="cuda")
    rs = torch.full((len(lengths),), -1, dtype=torch.int32, device="cuda")
    ws = torch.from_numpy(np.random.default_rng(3).permutation(wl["n_slots"])[:len(lengths)]
                          .astype(np.int32)).cuda()
    lib = gdn.load_library()
    s = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a_cw, _, keep_cw = gdn.make_prefill_args(cu, q, k, v, pool, rs, ws, H_qk=Hqk, H_v=Hv, g=gcw,
                                             beta=beta, scale=d ** -0.5)
    a_sc, _, keep_sc = gdn.make_prefill_args(cu, q, k, v, pool, rs, ws, H_qk=Hqk, H_v=Hv, g=g,
                                             beta=beta, scale=d ** -0.5)
    assert a_cw.decay_mode == gdn.DECAY_CHANNEL and a_sc.decay_mode == gdn.DECAY_HEAD

    def call(a):
        code = lib.gdn_prefill(ctypes.byref(a), s())
        if code:
            raise gdn.GdnError("gdn_prefill", code)

    def timed(a, reps):
        for _ in range(args.prefill_warmup):  # untimed: the first calls run slower
            call(a)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call(a)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(a_cw, args.prefill_reps)
    ms_sc = timed(a_sc, args.prefill_reps)
    flops = prefill_useful_flops(lengths, Hv, d, d)
    algo_bytes = (N * ((2 * Hqk * d + Hv * d) * 2 + Hv * d * 2 + Hv * d * 4 + Hv * 4)
                  + len(lengths) * Hv * d * d * 2)
    return dict(workload="prefill_varlen, channel-wise decay", tokens=N, rule="gated_delta",
                kernel="prefill_cw_kernel<bf16 state, bf16 act, 128, 128>",
                ms=round(ms, 3), tokens_per_s=round(N / (ms / 1e3), 1),
                scalar_gate_ms=round(ms_sc, 3), vs_scalar_gate=round(ms_sc / ms, 3),
                useful_tflops=round(flops / (ms / 1e3) / 1e12, 2),
                mfma_frac=round(flops / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                algorithmic_GBps=round(algo_bytes / (ms / 1e3) / 1e9, 1),
                hbm_frac=round(algo_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4))


def run_mixed(args, torch, gdn, syn):
    """448 decode requests plus 4 prefills of 8192 tokens (fused front-end) on
    one 1024-slot BF16 pool, 25% of requests reading a checkpoint slot (the
    prefills resume the conv window of their read slot and store the one they
    leave, in a conv pool of the same slots), decode rule gated_delta: one
    gdn_mixed call vs gdn_decode + gdn_prefill."""
    wl = syn.WORKLOADS["mixed"]
    Hqk, Hv, d = wl["H_qk"], wl["H_v"], wl["d_k"]
    nd, npf, L = wl["n_decode"], wl["n_prefill"], wl["prefill_len"]
    q, k, v, g, beta = (t.cuda() for t in syn.token_inputs(wl["index"], 1, nd, Hqk, Hv, d, d))
    pool = syn.state_pool(wl["index"], 0, wl["n_slots"], Hv, d, d, torch.bfloat16, on_device=True)
    drs, dws, prs, pws = (t.cuda() for t in syn.mixed_slots(wl["index"], nd, npf, wl["n_slots"]))
    cu = syn.cu_from_lengths([L] * npf).cuda()
    x = {kk: vv.cuda() for kk, vv in syn.frontend_inputs(wl["index"], 2, L * npf, Hqk, Hv, d, d, 4).items()}
    decs = {rule: gdn.make_decode_args(q, k, v, g, beta, pool, drs, dws, rule=rule)
            for rule in ("linear", "gated", "delta", "gated_delta")}
    cpool = syn.conv_pool(wl["index"], 0, wl["n_slots"], 2 * Hqk * d + Hv * d, 4, torch.bfloat16,
                          on_device=True)
    pa, po, pkeep = gdn.make_prefill_args(cu, x["q_raw"], x["k_raw"], x["v_raw"], pool, prs, pws,
                                          H_qk=Hqk, H_v=Hv, a_raw=x["a_raw"], b_raw=x["b_raw"],
                                          conv_wq=x["conv_wq"], conv_wk=x["conv_wk"],
                                          conv_wv=x["conv_wv"], conv_pool=cpool,
                                          conv_read_slot=prs, conv_write_slot=pws)
    lib = gdn.load_library()
    s = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    da = None  # the decode half's arguments, one update rule at a time

    def mixed():
        code = lib.gdn_mixed(ctypes.byref(da), ctypes.byref(pa), s())
        if code:
            raise gdn.GdnError("gdn_mixed", code)

    def separate():
        for fn, a in ((lib.gdn_decode, da), (lib.gdn_prefill, pa)):
            code = fn(ctypes.byref(a), s())
            if code:
                raise gdn.GdnError("separate", code)

    def timed(fn, reps):
        for _ in range(args.prefill_warmup):  # untimed: the first calls run slower
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    tokens = nd + npf * L
    rules = {}
    for rule, (a, _, _) in decs.items():
        da = a
        ms_mixed = timed(mixed, args.prefill_reps)
        ms_sep = timed(separate, args.prefill_reps)
        rules[rule] = dict(ms=round(ms_mixed, 3), tokens_per_s=round(tokens / (ms_mixed / 1e3), 1),
                           separate_ms=round(ms_sep, 3),
                           speedup_vs_separate=round(ms_sep / ms_mixed, 3))
    gd = rules["gated_delta"]
    return dict(workload="mixed", decode_requests=nd, prefill_tokens=npf * L,
                ms=gd["ms"], tokens_per_s=gd["tokens_per_s"], separate_ms=gd["separate_ms"],
                speedup_vs_separate=gd["speedup_vs_separate"], decode_rules=rules)


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
    # one thread, on the first 64 requests of layer 0 (scaled to the batch)
    _, keep = layers[0]
    q, k, v, g, beta, pool, rs, ws = keep[:8]
    n1 = 64
    f = lambda t: t[:n1].detach().to("cpu", torch.float64).numpy()
    hrs = rs[:n1].cpu().numpy()
    hpool = pool[torch.from_numpy(hrs).long().to(pool.device)].detach().to("cpu", torch.float64).numpy()
    own = np.arange(n1, dtype=np.int32)
    t0 = time.perf_counter()
    oracle.decode(f(q), f(k), f(v), f(g), f(beta), hpool, own, own, round_state=True, n_threads=1)
    t1 = (time.perf_counter() - t0) * B / n1
    del hpool
    model = "?"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=B / (per_layer * len(layers)), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"FP64 oracle on layers {picks} of {len(layers)} at B={B} (all request-heads), "
                       f"{per_layer:.2f}s per layer; tokens/s extrapolated to {len(layers)} layers",
                one_thread_value=B / (t1 * len(layers)),
                one_thread_sample=f"1 thread, {n1} requests of layer 0 ({t1 * n1 / B:.2f}s), "
                                  f"scaled to B={B} and {len(layers)} layers",
                cpu_model=model, nproc=os.cpu_count())


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-conv", action="store_true",
                    help="skip the decode-side conv and the channel-wise decay measurements")
    ap.add_argument("--no-b64", action="store_true", help="skip the B=64 decode leg")
    ap.add_argument("--no-q8", action="store_true", help="skip the 8-bit state decode leg")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--prefill-warmup", type=int, default=10,
                    help="untimed calls before the prefill and mixed timings")
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

    copy = run_copy(args, torch)
    log(f"copy: {copy}")
    dec, layers = run_decode(args, torch, gdn, syn)
    achieved = dec["bytes_per_launch"] / (dec["avg_launch_us"] / 1e6) / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=recorded_traffic(),
                    copy_GBps=copy["GBps"], frac_of_copy=round(achieved / copy["GBps"], 4),
                    kernel="decode_kernel<bf16 state, bf16 act, 128, 128>",
                    per_launch_bytes=dec["bytes_per_launch"],
                    avg_launch_us=round(dec["avg_launch_us"], 2))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(args, torch, layers, syn)
    conv = None
    if not args.no_conv:
        conv = run_conv(args, torch, gdn, syn, layers)
        conv["small_batch"] = run_conv_small(args, torch, gdn, syn)
        log(f"conv: {conv}")
    decode_cw = None
    if not args.no_conv:
        decode_cw = run_decode_cw(args, torch, gdn, syn, layers)
        log(f"decode, channel-wise decay: {decode_cw}")
    decode_q8 = state_convert = None
    if not args.no_q8:
        decode_q8 = [run_decode_q8(args, torch, gdn, syn, layers, n_hi) for n_hi in (32, 0)]
        log(f"decode, 8-bit state: {decode_q8}")
        state_convert = run_convert(args, torch, gdn, syn, layers)
        log(f"state convert: {state_convert}")
        torch.cuda.empty_cache()
    prefill = None
    if not args.no_prefill:
        del layers[:]
        torch.cuda.empty_cache()
    decode_b64 = None
    if not args.no_b64:
        decode_b64 = run_decode_b64(args, torch, gdn, syn)
        log(f"decode B=64: {decode_b64}")
        torch.cuda.empty_cache()
    if not args.no_prefill:
        torch.cuda.empty_cache()
        prefill = run_prefill(args, torch, gdn, syn)
        log(f"prefill: {prefill}")
    prefill_cw = None
    if not args.no_prefill:
        torch.cuda.empty_cache()
        prefill_cw = run_prefill_cw(args, torch, gdn, syn)
        log(f"prefill, channel-wise decay: {prefill_cw}")
    mixed = None
    if not args.no_prefill:
        torch.cuda.empty_cache()
        mixed = run_mixed(args, torch, gdn, syn)
        log(f"mixed: {mixed}")
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
        "copy": copy,
        "cpu_baseline": cpu,
        "decode_b64": decode_b64,
        "conv_decode": conv,
        "decode_channel_decay": decode_cw,
        "decode_q8_state": decode_q8,
        "state_convert": state_convert,
        "prefill": prefill,
        "prefill_channel_decay": prefill_cw,
        "mixed": mixed,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
