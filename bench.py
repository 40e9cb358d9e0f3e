#!/usr/bin/env python3
"""Throughput of the BitLinear hot path on one MI355X.

Headline workload (``value``): decode at M = 1 over the four 2B-class BitLinear
shapes (fused QKV 2560->3840, O 2560->2560, fused up/gate 2560->13824, down
6912->2560), for 30 layers whose packed weights sit at 30 distinct HBM
addresses (521 MB per step, twice the 256 MB Infinity Cache, so every step
streams its weights from HBM).  One step = for every layer and matrix:
per-token absmax quantisation of that matrix's input, then the ternary
product with rescale.  Weights are quantised and packed once, before timing
(the method packs them offline).  Metric: packed-weight bytes per second.

Also measured on the same line (``extra``): the 70B-class layer at M = 1
(2-bit and base-3 layouts) and M = 16 / 128, the 30-layer 2B-class decoder
stack at M = 64 in tokens/s, and the 3B-class prefill GEMM at M = 512 in
TOPS; plus the roofline of the dominant kernel and the CPU oracle timed on a
bounded sample on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector peak
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
I8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, TOP/s
METRIC = "BitLinear weight GB/s (% HBM peak) at M=1; TOPS (% int8 MFMA peak) at M=512"
WARM_MS = 20.0   # replays of the same graph before the timed ones in the non-headline sections


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--no-extra", action="store_true", help="skip the 70B / prefill lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-separate-stack", action="store_true",
                    help="skip the layer stack timed with separate product and glue calls")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", default="",
                    help="comma-separated sections to run instead of the whole line (for "
                         "profiling): decode, xl, stack, prefill, variants, backward, ceilings, "
                         "cpu")
    ap.add_argument("--graph-only", action="store_true",
                    help="time only the graph replays (no eager or GEMV-alone runs), so that "
                         "a kernel trace of the run holds graph-replayed dispatches only")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy kernel (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def time_loop(fn, iters, warmup):
    """Average ms per call of fn() over `iters` calls, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def graph_time(fn, replays, warmup, min_warm_ms=0.0):
    """Capture fn() (a fixed sequence of launches) in one HIP graph and return
    the average ms per replay over `replays` back-to-back replays (HIP events
    on the replay stream).  Graph replay takes the Python and launch-queue
    overhead out of the timed region; every kernel still runs as launched.
    `warmup` replays precede the timed ones, and more until at least
    `min_warm_ms` of replays have run (at most 400), so that the clocks have
    settled after the host-side set-up of a section: the first replays of a
    freshly captured graph run 5-8% slower."""
    import torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fn()                               # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fn()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    if min_warm_ms > 0:
        done_ms, n = 0.0, 0
        while done_ms < min_warm_ms and n < 400:
            start.record(cur)
            for _ in range(4):
                graph.replay()
            end.record(cur)
            torch.cuda.synchronize()
            done_ms += start.elapsed_time(end)
            n += 4
    start.record(cur)
    for _ in range(replays):
        graph.replay()
    end.record(cur)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / replays


def decode_workload(layers):
    """Quantise the four decode matrices once; replicate the packed weights to
    `layers` distinct buffers; inputs resident in HBM."""
    import torch
    from ternary_weight_linear_absmax_amd import bitlinear as bl
    from ternary_weight_linear_absmax_amd import inputs
    mats = []
    for i in range(len(inputs.DECODE_SHAPES)):
        name, w, x = inputs.decode(i, m=1)
        n, k = w.shape
        packed, gamma = bl.quantize_weights(to_dev(w))
        xd = to_dev(x)
        copies = [packed] + [packed.clone() for _ in range(layers - 1)]
        xq, scale, rowsum = bl.quantize_act(xd)
        y = torch.empty((1, n), dtype=torch.float32, device="cuda")
        mats.append(dict(name=name, n=n, k=k, x=xd, copies=copies, gamma=gamma, xq=xq,
                         scale=scale, rowsum=rowsum, y=y, bytes=packed.numel()))
    torch.cuda.synchronize()
    return mats


def sections(args):
    """Sections to run: the whole line by default, or the --only list."""
    every = ["decode", "ceilings", "xl", "stack", "prefill", "variants", "backward", "cpu"]
    if not args.only:
        out = list(every)
        if args.no_extra:
            out = [x for x in out if x in ("decode", "cpu")]
        if args.no_cpu:
            out.remove("cpu")
        return out
    want = [x.strip() for x in args.only.split(",") if x.strip()]
    bad = [x for x in want if x not in every]
    if bad:
        raise SystemExit(f"unknown section(s) {bad}; choose from {every}")
    return want


def measure_decode(args):
    """Headline: the decode step (one bitlinear_quantize_forward launch per
    matrix and layer), graph-replayed; returns the line's core fields."""
    import torch
    from ternary_weight_linear_absmax_amd import bitlinear as bl
    mats = decode_workload(args.layers)
    step_bytes = sum(m["bytes"] for m in mats) * args.layers
    log(f"decode workload ready: {step_bytes / 1e6:.1f} MB packed per step")

    def step():
        # per matrix: quantise its input and multiply (bitlinear_quantize_forward)
        for layer in range(args.layers):
            for m in mats:
                bl.quantize_forward(m["x"], m["copies"][layer], m["gamma"], m["n"], y=m["y"],
                                    xq=m["xq"], scale=m["scale"], rowsum=m["rowsum"])

    # one step = one replay of the captured step (120 launches at 30 layers)
    ms_step = graph_time(step, args.steps, args.warmup)
    ms_step_eager = None if args.graph_only else time_loop(step, max(2, args.steps // 10), 1)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    eager = "" if ms_step_eager is None else f" (eager launches: {ms_step_eager * 1e3:.1f} us)"
    log(f"decode step {ms_step * 1e3:.1f} us{eager} -> {value:.1f} GB/s")

    # dominant kernel: the step is one launch per matrix (one-token quantisation
    # fused into the 2-bit GEMV), so its per-launch time is the step's
    launches = args.layers * len(mats)
    us_per_launch = ms_step * 1e3 / launches
    bytes_per_launch = step_bytes / launches
    achieved = bytes_per_launch / (us_per_launch * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(),
                "kernel": "gemv2_kernel<1,CPL,ST,true,bf16> (decode, M=1, activation "
                          "quantisation inside); per-launch time = graph replay / launches",
                "avg_launch_us": round(us_per_launch, 3),
                "algorithmic_bytes_per_launch": int(bytes_per_launch),
                "per_matrix_bytes": {m["name"]: m["bytes"] for m in mats}}

    if args.graph_only:
        return dict(value=value, ms_step=ms_step, ms_step_eager=None, step_bytes=step_bytes,
                    roofline=roofline, launches=launches)

    # the same GEMV on pre-quantised activations, timed alone over the same rotation
    def gemv_only():
        for layer in range(args.layers):
            for m in mats:
                bl.forward(m["xq"], m["scale"], m["rowsum"], m["copies"][layer], m["gamma"],
                           m["n"], m["k"], y=m["y"])
    ms_gemv = graph_time(gemv_only, args.steps, args.warmup)
    roofline["prequantised_gemv_us_per_launch"] = round(ms_gemv * 1e3 / launches, 3)
    log(f"decode per launch: {us_per_launch:.2f} us with quantisation, "
        f"{ms_gemv * 1e3 / launches:.2f} us GEMV alone")

    # a few tokens at once (M = 2 and 4, pre-quantised, the path AUTO takes:
    # the GEMV on these matrices), the same 30-layer rotation
    multi = {}
    for mt in (2, 4):
        g = torch.Generator(device="cuda").manual_seed(90 + mt)
        for m in mats:
            xm = torch.randn((mt, m["k"]), device="cuda", generator=g).to(torch.bfloat16)
            m["xqM"], m["scM"], m["rsM"] = bl.quantize_act(xm)
            m["yM"] = torch.empty((mt, m["n"]), dtype=torch.float32, device="cuda")

        def few_tokens():
            for layer in range(args.layers):
                for m in mats:
                    bl.forward(m["xqM"], m["scM"], m["rsM"], m["copies"][layer], m["gamma"],
                               m["n"], m["k"], y=m["yM"])
        ms_m = graph_time(few_tokens, args.steps, args.warmup)
        multi[f"decode_M{mt}"] = {
            "us_per_step": round(ms_m * 1e3, 1),
            "GB/s": round(step_bytes / (ms_m * 1e-3) / 1e9, 1),
            "hbm_frac": round(step_bytes / (ms_m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "paths": sorted({bl.forward_path(mt, m["n"], m["k"]) for m in mats})}
        log(f"decode M={mt}: {ms_m * 1e3:.1f} us per step")
    return dict(value=value, ms_step=ms_step, ms_step_eager=ms_step_eager, step_bytes=step_bytes,
                roofline=roofline, launches=launches, multi=multi)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; run with --gpus 1 "
                          "(sharding over several GPUs is described, not implemented)"}))
        sys.exit(2)

    import torch
    from ternary_weight_linear_absmax_amd import bitlinear as bl

    if args.calibrate_copy:
        calibrate_copy()
        return
    bl.load()
    dev_name = torch.cuda.get_device_name(0)
    log(f"device {dev_name}")
    todo = sections(args)
    log(f"sections: {', '.join(todo)}")

    dec = measure_decode(args) if "decode" in todo else None
    extra = dict(dec.get("multi", {})) if dec else {}
    ceil = measure_ceilings(args) if "ceilings" in todo else None
    if ceil:
        extra["ceilings"] = ceil
    if "xl" in todo:
        extra.update(measure_xl(args))
    if "stack" in todo:
        extra.update(measure_stack(separate=not args.no_separate_stack))
    roofline_prefill = None
    if "prefill" in todo:
        pre, roofline_prefill = measure_prefill(ceil)
        extra.update(pre)
    if "variants" in todo:
        extra.update(measure_variants())
    if "backward" in todo:
        extra.update(measure_backward())
    cpu = cpu_baseline(args.cpu_seconds) if "cpu" in todo else None
    if dec and ceil:
        dec["roofline"]["frac_of_measured_read_ceiling"] = round(
            dec["roofline"]["achieved"] / ceil["hbm_read_stream_GB/s"], 4)
        floor = ceil["decode_plain_read_us_per_launch"]
        dec["roofline"]["plain_read_same_launches_us"] = floor

    out = {
        "metric": METRIC,
        "value": round(dec["value"], 2) if dec else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_step"], 4) if dec else None,
        "ms_per_step_eager_launch": (round(dec["ms_step_eager"], 4)
                                     if dec and dec["ms_step_eager"] is not None else None),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": "decode M=1, 2B-class BitLinear shapes (QKV 2560x3840, O 2560x2560, "
                        "up/gate 2560x13824, down 6912x2560), %d layers of distinct packed "
                        "weights; per matrix: absmax int8 quantisation + ternary GEMV + rescale, "
                        "the step captured in a HIP graph" % args.layers,
            "M": 1,
            "layers": args.layers,
            "packed_bytes_per_step": dec["step_bytes"] if dec else None,
            "hbm_frac": round(dec["value"] / HBM_PEAK_GBS, 4) if dec else None,
            "device": dev_name,
            "sections": todo,
        },
        "roofline": dec["roofline"] if dec else None,
        "roofline_prefill": roofline_prefill,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


CEILINGS_LIB = os.path.join(ROOT, "ternary_weight_linear_absmax_amd", "libbitlinear_ceilings.so")


def _ceilings_lib():
    import ctypes
    if not os.path.exists(CEILINGS_LIB):
        raise RuntimeError(f"{CEILINGS_LIB} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(CEILINGS_LIB)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.blc_read_stream.argtypes = [p, i64, i32, p, p]
    lib.blc_read_stream.restype = i32
    lib.blc_mfma_i8_ops.argtypes = [i32, i32]
    lib.blc_mfma_i8_ops.restype = i64
    lib.blc_mfma_i8_loop.argtypes = [i32, i32, p, p]
    lib.blc_mfma_i8_loop.restype = i32
    lib.blc_empty.argtypes = [p]
    lib.blc_empty.restype = i32
    lib.blc_lds_mix.argtypes = [i32, i32, i32, i32, p, i64, p, p]
    lib.blc_lds_mix.restype = i32
    return lib


def measure_ceilings(args):
    """Measured ceilings of this device (libbitlinear_ceilings.so): a plain
    HBM read stream (1 GiB of 16-byte non-temporal loads), the same plain read
    over the decode step's launches (each decode matrix's byte count, from 30
    distinct addresses, graph-replayed like the decode step) and over the
    70B-class matrix size, an empty kernel per graph node, and an int8
    matrix-core loop with no memory traffic."""
    import ctypes
    import torch
    from ternary_weight_linear_absmax_amd import inputs
    from ternary_weight_linear_absmax_amd import bitlinear as bl
    lib = _ceilings_lib()
    sink = torch.zeros((4,), dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(sink.data_ptr())

    def st():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def chk(rc):
        if rc != 0:
            raise RuntimeError(f"ceiling kernel failed ({rc})")
    out = {}
    gib = 1 << 30
    buf = torch.empty((gib,), dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    bp = buf.data_ptr()
    best = 0.0
    for blocks in (1024, 2048, 4096, 8192):
        ms = graph_time(lambda: chk(lib.blc_read_stream(ctypes.c_void_p(bp), gib, blocks, sp,
                                                        st())), 10, 2)
        gbs = gib / (ms * 1e-3) / 1e9
        out[f"read_stream_1GiB_{blocks}_blocks_GB/s"] = round(gbs, 1)
        best = max(best, gbs)
    out["hbm_read_stream_GB/s"] = round(best, 1)
    out["hbm_read_stream_frac_of_peak"] = round(best / HBM_PEAK_GBS, 4)
    log(f"ceiling: HBM read stream {best:.0f} GB/s")

    # the decode step's launch pattern with a plain read in place of each GEMV
    sizes = [bl.packed_bytes(n, k) for (_, k, n) in inputs.DECODE_SHAPES]
    layers = args.layers
    offs = []
    off = 0
    for _ in range(layers):
        for b in sizes:
            offs.append((off, b))
            off += (b + 4095) // 4096 * 4096
    assert off <= gib

    def plain_step():
        for o, b in offs:
            chk(lib.blc_read_stream(ctypes.c_void_p(bp + o), b, 1024, sp, st()))
    ms = graph_time(plain_step, 20, 3)
    out["decode_plain_read_us_per_launch"] = round(ms * 1e3 / len(offs), 3)
    out["decode_plain_read_GB/s"] = round(sum(sizes) * layers / (ms * 1e-3) / 1e9, 1)
    log(f"ceiling: plain read of the decode step {ms * 1e3:.1f} us "
        f"({ms * 1e3 / len(offs):.2f} us per launch)")
    for i, (name, k, n) in enumerate(inputs.DECODE_SHAPES):
        def one():
            for layer in range(layers):
                o, b = offs[layer * len(sizes) + i]
                chk(lib.blc_read_stream(ctypes.c_void_p(bp + o), b, 1024, sp, st()))
        ms = graph_time(one, 20, 3)
        out[f"decode_plain_read_{name}_us"] = round(ms * 1e3 / layers, 3)
    xl_bytes = bl.packed_bytes(28672, 8192)
    copies = gib // ((xl_bytes + 4095) // 4096 * 4096)
    copies = min(copies, 10)
    stride = (xl_bytes + 4095) // 4096 * 4096
    for blocks in (2048, 4096):
        def xl_read():
            for c in range(copies):
                chk(lib.blc_read_stream(ctypes.c_void_p(bp + c * stride), xl_bytes, blocks, sp,
                                        st()))
        ms = graph_time(xl_read, 20, 3) / copies
        out[f"xl_plain_read_{blocks}_blocks_us"] = round(ms * 1e3, 2)
    out["xl_plain_read_us"] = min(out["xl_plain_read_2048_blocks_us"],
                                  out["xl_plain_read_4096_blocks_us"])
    del buf
    torch.cuda.empty_cache()

    def empties():
        for _ in range(120):
            chk(lib.blc_empty(st()))
    ms = graph_time(empties, 20, 3)
    out["empty_kernel_graph_node_us"] = round(ms * 1e3 / 120, 3)
    log(f"ceiling: empty kernel {ms * 1e3 / 120:.2f} us per graph node")

    iters, blocks = 2000, 1024
    ms = graph_time(lambda: chk(lib.blc_mfma_i8_loop(iters, blocks, sp, st())), 5, 1)
    tops = lib.blc_mfma_i8_ops(iters, blocks) / (ms * 1e-3) / 1e12
    out["mfma_i8_loop_TOPS"] = round(tops, 1)
    out["mfma_i8_loop_frac_of_peak"] = round(tops / I8_PEAK_TOPS, 4)
    log(f"ceiling: int8 matrix-core loop {tops:.0f} TOPS")
    out.update(measure_lds_mix(lib, chk, st, sp))
    return out


def measure_lds_mix(lib, chk, st, sp):
    """LDS traffic in the tiled GEMM's patterns, two 512-thread blocks per CU
    (blc_lds_mix): the fragment reads of four waves alone, 16-byte LDS writes
    of the other four waves alone (as ds_write_b128, or as direct
    global-to-LDS loads from an 8 MiB window), and both together.  Run
    together, the reads and writes overlap fully when the time is the longer
    of the two alone and not at all when it is their sum; `overlap` is
    (alone_r + alone_w - together) / min(alone_r, alone_w)."""
    import ctypes
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    window = 8 << 20
    src = torch.ones((window,), dtype=torch.uint8, device="cuda")
    srcp = ctypes.c_void_p(src.data_ptr())
    it_r = 2000
    out = {}

    def t(mode, ir, iw):
        return graph_time(lambda: chk(lib.blc_lds_mix(mode, ir, iw, blocks, srcp, window, sp,
                                                      st())), 5, 1) * 1e3
    read_us = t(0, it_r, 0)
    per_cu_read = 2 * it_r * 16384 / (read_us * 1e-6) / 1e9
    out["lds_read_alone_us"] = round(read_us, 1)
    out["lds_read_GB/s_per_CU"] = round(per_cu_read, 1)
    for name, mode, it_w in (("ds_write_b128", 1, 4000), ("direct_load", 2, 2400)):
        w_us = t(mode, 0, it_w)
        both_us = t(mode, it_r, it_w)
        ov = (read_us + w_us - both_us) / min(read_us, w_us)
        out[f"lds_{name}_alone_us"] = round(w_us, 1)
        out[f"lds_{name}_GB/s_per_CU"] = round(2 * it_w * 4096 / (w_us * 1e-6) / 1e9, 1)
        out[f"lds_read_with_{name}_us"] = round(both_us, 1)
        out[f"lds_read_with_{name}_overlap"] = round(ov, 3)
        log(f"ceiling: LDS fragment reads {read_us:.0f} us alone, {name} {w_us:.0f} us alone, "
            f"{both_us:.0f} us together (overlap {ov:.2f})")
    del src
    return out


def measure_xl(args):
    """The 70B-class layer (rotating 10 copies of each matrix, 587 MB, so the
    weights stream from HBM) at M = 1, 16, 128 and in base-3 at M = 1, plus
    the weight quantiser on the same matrices."""
    import torch
    from ternary_weight_linear_absmax_amd import bitlinear as bl
    from ternary_weight_linear_absmax_amd import inputs
    extra = {}
    copies_n = 10
    for si, (name, k, n) in enumerate(inputs.XL_SHAPES):
        _, w, x = inputs.xl(si, m=128)
        wd = to_dev(w)
        p2, g2 = bl.quantize_weights(wd)
        p3, g3 = bl.quantize_weights(wd, bl.BL_PACK3)
        # weight quantiser (offline step): gamma pass + packing pass over W;
        # two copies of W alternate so that neither is left in the last-level
        # cache by the previous call
        ws_w = torch.empty((bl.quantize_weights_workspace_bytes(n, k),), dtype=torch.uint8,
                           device="cuda")
        wd2 = wd.clone()
        for lay, (pk, gk), tag in ((bl.BL_PACK2, (p2, g2), "pack2"), (bl.BL_PACK3, (p3, g3), "pack3")):
            def quant_two():
                bl.quantize_weights(wd, lay, out=(pk, gk), workspace=ws_w)
                bl.quantize_weights(wd2, lay, out=(pk, gk), workspace=ws_w)
            ms_q = graph_time(quant_two, 5, 1) / 2
            moved = 2 * wd.numel() * wd.element_size() + pk.numel()
            extra[f"xl_{name}_quantize_weights_{tag}"] = {
                "us": round(ms_q * 1e3, 1), "GB/s": round(moved / (ms_q * 1e-3) / 1e9, 1),
                "hbm_frac": round(moved / (ms_q * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "bytes": moved}
            log(f"xl {name} quantize_weights {tag}: {ms_q * 1e3:.1f} us")
        del wd, wd2, ws_w
        c2 = [p2] + [p2.clone() for _ in range(copies_n - 1)]
        c3 = [p3] + [p3.clone() for _ in range(copies_n - 1)]
        xq, scale, rowsum = bl.quantize_act(to_dev(x))
        for m in inputs.XL_MS:
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")

            def fwd2():
                for c in c2:
                    bl.forward(xq[:m], scale[:m], rowsum[:m], c, g2, n, k, y=y)
            ms = graph_time(fwd2, 20, 3, WARM_MS) / copies_n
            gbs = p2.numel() / (ms * 1e-3) / 1e9
            tops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            extra[f"xl_{name}_M{m}_pack2"] = {
                "K": k, "N": n, "M": m, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "TOPS": round(tops, 2),
                "i8_frac": round(tops / I8_PEAK_TOPS, 4),
                "path": bl.forward_path(m, n, k)}
            log(f"xl {name} M={m} pack2: {ms * 1e3:.1f} us {gbs:.0f} GB/s {tops:.1f} TOPS")
            if m == 1:
                def fwd3():
                    for c in c3:
                        bl.forward(xq[:1], scale[:1], rowsum[:1], c, g3, n, k,
                                   layout=bl.BL_PACK3, y=y)
                ms3 = graph_time(fwd3, 20, 3, WARM_MS) / copies_n
                gbs3 = p3.numel() / (ms3 * 1e-3) / 1e9
                extra[f"xl_{name}_M1_pack3"] = {
                    "K": k, "N": n, "M": 1, "us": round(ms3 * 1e3, 2), "GB/s": round(gbs3, 1),
                    "hbm_frac": round(gbs3 / HBM_PEAK_GBS, 4),
                    "trits_per_s": round(n * k / (ms3 * 1e-3), 1)}
                log(f"xl {name} M=1 pack3: {ms3 * 1e3:.1f} us {gbs3:.0f} GB/s")
        del c2, c3
        torch.cuda.empty_cache()
    return extra


def measure_prefill(ceil):
    """The 3B-class prefill products at M = 512 (packed weights 6.9 MB: they
    stay in the Infinity Cache), the product alone and with the activation
    quantiser; the int8 library GEMM (torch._int_mm, unpacked int8 weights)
    on the same shapes for context.  Returns (entries, roofline object of the
    slower shape's product)."""
    import torch
    from ternary_weight_linear_absmax_amd import bitlinear as bl
    from ternary_weight_linear_absmax_amd import inputs
    extra = {}
    reps = 10
    worst = None
    for si, (name, k, n) in enumerate(inputs.PREFILL_SHAPES):
        _, w, x = inputs.prefill(si)
        packed, gamma = bl.quantize_weights(to_dev(w))
        xd = to_dev(x)
        xq, scale, rowsum = bl.quantize_act(xd)
        m = x.shape[0]
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")

        def fwd():
            for _ in range(reps):
                bl.forward(xq, scale, rowsum, packed, gamma, n, k, y=y)
        ms = graph_time(fwd, 20, 3, WARM_MS) / reps
        tops = 2.0 * m * n * k / (ms * 1e-3) / 1e12

        def full():
            for _ in range(reps):
                bl.quantize_act(xd)
                bl.forward(xq, scale, rowsum, packed, gamma, n, k, y=y)
        ms_full = graph_time(full, 20, 3, WARM_MS) / reps
        ent = {"K": k, "N": n, "M": m, "us": round(ms * 1e3, 2), "TOPS": round(tops, 2),
               "i8_frac": round(tops / I8_PEAK_TOPS, 4),
               "us_with_act_quant": round(ms_full * 1e3, 2),
               "TOPS_with_act_quant": round(2.0 * m * n * k / (ms_full * 1e-3) / 1e12, 2),
               "splits_workspace_bytes": bl.forward_workspace_bytes(m, n, k)}
        if ceil:
            ent["frac_of_measured_mfma_ceiling"] = round(tops / ceil["mfma_i8_loop_TOPS"], 4)
        # context: the int8 library GEMM on unpacked int8 operands
        try:
            a8 = xq
            b8 = bl.unpack_weights(packed, n, k).t()     # [K, N] view of the trits
            b8c = b8.contiguous()
            ms_lib = time_loop(lambda: torch._int_mm(a8, b8c), 20, 3)
            ent["library_int8_gemm_us"] = round(ms_lib * 1e3, 2)
        except Exception as e:                             # library path missing on this build
            ent["library_int8_gemm_us"] = f"unavailable: {type(e).__name__}"
        extra[f"prefill_{name}_M512"] = ent
        log(f"prefill {name}: {ms * 1e3:.1f} us {tops:.1f} TOPS")
        if worst is None or ms > worst[0]:
            worst = (ms, name, m, n, k, tops)
    ms, name, m, n, k, tops = worst
    roof = {"bound": "mfma", "achieved": round(tops, 1), "peak": I8_PEAK_TOPS, "unit": "TOP/s",
            "frac": round(tops / I8_PEAK_TOPS, 4), "traffic": None,
            "kernel": f"tiled int8 GEMM, prefill {name} M={m} N={n} K={k} (the slower of the "
                      f"two 3B-class shapes; per-launch time = graph replay / launches, "
                      f"including a split-k finish where the shape splits)",
            "avg_launch_us": round(ms * 1e3, 3), "algorithmic_ops_per_launch": 2 * m * n * k}
    if ceil:
        roof["frac_of_measured_mfma_ceiling"] = round(tops / ceil["mfma_i8_loop_TOPS"], 4)
    return extra, roof


def measure_backward():
    """Input gradient through BitLinear (straight-through estimators) on the
    3B-class prefill matrices at M = 512: 2 M N K flops, against the fp32
    vector peak and, as run, against the bf16 matrix-core peak (bf16
    gradients: one bf16 MFMA per product; fp32 gradients: three, the gradient
    split in three bf16 parts)."""
    import torch
    from ternary_weight_linear_absmax_amd import bitlinear as bl
    from ternary_weight_linear_absmax_amd import inputs
    out = {}
    reps = 5
    for si, (name, k, n) in enumerate(inputs.PREFILL_SHAPES):
        _, w, _ = inputs.prefill(si)
        packed, gamma = bl.quantize_weights(to_dev(w))
        m = 512
        g32 = torch.randn((m, n), device="cuda") * 1e-3
        gx = torch.empty((m, k), dtype=torch.float32, device="cuda")
        for tag, gy, parts in (("", g32.to(torch.bfloat16), 1), ("_fp32grad", g32, 3)):
            def bwd():
                for _ in range(reps):
                    bl.backward_input(gy, packed, gamma, k, grad_x=gx)
            ms = graph_time(bwd, 10, 2, WARM_MS) / reps
            tflops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            out[f"backward_input_{name}_M512{tag}"] = {
                "K": k, "N": n, "M": m, "grad_dtype": "bf16" if parts == 1 else "fp32",
                "us": round(ms * 1e3, 2), "TFLOP/s": round(tflops, 2),
                "fp32_equiv_frac": round(tflops / FP32_PEAK_TFLOPS, 4),
                "bf16_mfma_TFLOP/s": round(parts * tflops, 1),
                "bf16_mfma_frac": round(parts * tflops / BF16_PEAK_TFLOPS, 4)}
            log(f"backward input {name}{tag}: {ms * 1e3:.1f} us {tflops:.1f} TFLOP/s")
    return out


def measure_variants():
    """The variants on their natural shapes: sign-binarised 70B-class weights
    at M = 1 (10 rotating copies) and 4-bit activations on the 3B-class
    prefill product at M = 512 (quantiser + product)."""
    import torch
    from ternary_weight_linear_absmax_amd import bitlinear as bl
    from ternary_weight_linear_absmax_amd import inputs
    out = {}
    name, k, n = inputs.XL_SHAPES[0]
    _, w, x = inputs.xl(0, m=1)
    wd = to_dev(w)
    pb, beta = bl.quantize_weights(wd, binary=True)
    del wd
    copies = [pb] + [pb.clone() for _ in range(9)]
    xq, scale, rowsum = bl.quantize_act(to_dev(x))
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")

    def fwd():
        for c in copies:
            bl.forward(xq, scale, rowsum, c, beta, n, k, y=y)
    ms = graph_time(fwd, 20, 3, WARM_MS) / len(copies)
    gbs = pb.numel() / (ms * 1e-3) / 1e9
    out[f"binary_weights_xl_{name}_M1"] = {"K": k, "N": n, "M": 1, "us": round(ms * 1e3, 2),
                                            "GB/s": round(gbs, 1),
                                            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    log(f"binary weights xl {name} M=1: {ms * 1e3:.1f} us {gbs:.0f} GB/s")
    del copies
    name, k, n = inputs.PREFILL_SHAPES[0]
    _, w, x = inputs.prefill(0)
    packed, gamma = bl.quantize_weights(to_dev(w))
    xd = to_dev(x)
    m = x.shape[0]
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    reps = 10

    def full4():
        for _ in range(reps):
            q4, s4, r4 = bl.quantize_act(xd, bits=4)
            bl.forward(q4, s4, r4, packed, gamma, n, k, y=y)
    ms = graph_time(full4, 20, 3, WARM_MS) / reps
    tops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    out[f"act4_prefill_{name}_M512"] = {"K": k, "N": n, "M": m, "us_with_act_quant": round(ms * 1e3, 2),
                                         "TOPS_with_act_quant": round(tops, 2),
                                         "i8_frac": round(tops / I8_PEAK_TOPS, 4)}
    log(f"4-bit activations prefill {name}: {ms * 1e3:.1f} us {tops:.1f} TOPS")
    return out


def measure_stack(layers=30, m=64, separate=True):
    """The 2B-class layer stack (hidden 2560, 20/5 heads of 128, FFN 6912,
    squared ReLU, RMSNorm before every BitLinear), M tokens decoded at
    sequence position 0, one step = all layers, captured in one HIP graph.
    Weights: bf16 N(0, 0.02) drawn on the GPU with torch's generator seeded
    4000 + 10 * layer + matrix index; x0 ~ N(0, 1)."""
    import torch
    from ternary_weight_linear_absmax_amd import stack as st
    gen = torch.Generator(device="cuda")

    def weights(layer):
        out = {}
        for i, name in enumerate(st.MATRICES):
            gen.manual_seed(4000 + 10 * layer + i)
            out[name] = (torch.randn(st.SHAPES[name], generator=gen, device="cuda")
                         * 0.02).to(torch.bfloat16)
        return out

    stack = st.DecoderStack(weights, layers, m)
    gen.manual_seed(4999)
    x0 = torch.randn((m, st.HIDDEN), device="cuda", generator=gen)

    def step():
        stack.x.copy_(x0)
        stack.step()
    pb = stack.packed_bytes()
    from ternary_weight_linear_absmax_amd import bitlinear as bl
    ops = 2.0 * m * sum(st.SHAPES[n][0] * st.SHAPES[n][1] for n in st.MATRICES) * layers
    out = {}
    # fused: four product + glue calls per layer, two launches each (every
    # product here runs on the tiled GEMM, whose split partial sums the glue
    # kernel finishes); separate calls: four quantiser launches and four
    # products, each with a finish launch when it splits its k range
    split = sum(bl.forward_workspace_bytes(m, *st.SHAPES[n]) > 0 for n in st.MATRICES)
    variants = [(True, "stack_2B_M64", 8)]
    if separate:
        variants.append((False, "stack_2B_M64_separate_calls", 8 + split))
    for fused, name, per_layer in variants:
        stack.fused = fused
        ms = graph_time(step, 20, 3, WARM_MS)
        out[name] = {
            "layers": layers, "M": m, "us_per_step": round(ms * 1e3, 1),
            "tokens_per_s": round(m / (ms * 1e-3), 1), "packed_bytes": pb,
            "GB/s": round(pb / (ms * 1e-3) / 1e9, 1), "TOPS": round(ops / (ms * 1e-3) / 1e12, 2),
            "launches_per_step": per_layer * layers + 1}
        log(f"{name} {layers} layers M={m}: {ms * 1e3:.1f} us/step, "
            f"{m / (ms * 1e-3):.0f} tokens/s")
    del stack
    torch.cuda.empty_cache()

    # one token through the same layers with the glue as the products'
    # prologue / epilogue (RMSNorm + quantisation inside the GEMV, relu^2 * up
    # in the up/gate epilogue): four launches per layer
    stack1 = st.DecoderStack(weights, layers, 1, norm=True)
    gen.manual_seed(4998)
    x1 = torch.randn((1, st.HIDDEN), device="cuda", generator=gen)

    def step1():
        stack1.x.copy_(x1)
        stack1.step()
    ms = graph_time(step1, 20, 3, WARM_MS)
    pb1 = stack1.packed_bytes()
    out["stack_2B_M1_norm_prologue"] = {
        "layers": layers, "M": 1, "us_per_step": round(ms * 1e3, 1),
        "tokens_per_s": round(1 / (ms * 1e-3), 1), "packed_bytes": pb1,
        "GB/s": round(pb1 / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(pb1 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "launches_per_step": 4 * layers + 3}   # + input copy, last residual, output copy
    log(f"stack_2B_M1_norm_prologue {layers} layers M=1: {ms * 1e3:.1f} us/step")
    del stack1
    torch.cuda.empty_cache()
    return out


COPY_BYTES = 1 << 30


def calibrate_copy():
    """A plain copy of known size for the hardware byte counters: torch's
    elementwise negation reads COPY_BYTES and writes COPY_BYTES once each."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "torch.neg float32", "read_bytes": COPY_BYTES,
                      "write_bytes": COPY_BYTES, "dispatches": 3}), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_decode_m1_traffic.txt")
TRAFFIC_SOURCES = ["ternary_weight_linear_absmax_amd/csrc/gemv.hip",
                   "ternary_weight_linear_absmax_amd/csrc/internal.h"]


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode GEMV launch from the committed counter summary, or
    None when it is missing or was taken on other kernel sources."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    fields[key.strip()] = val.strip()
        if fields.get("sources_sha256_16") != sources_digest():
            return None
        return int(float(fields["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _split_rows(fn, rows, threads):
    """fn(r0, r1) over row ranges on `threads` host threads (the oracle's
    ctypes calls release the GIL)."""
    import concurrent.futures
    bounds = np.linspace(0, rows, threads + 1).astype(int)
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda i: fn(bounds[i], bounds[i + 1]), range(threads)))


def cpu_baseline(seconds):
    """The oracle, untuned, on this host.  Headline value: the decode
    workload's per-matrix chain (absmax quantisation, exact int32 product,
    rescale) at M = 1 on one thread, repeated over the four shapes until
    `seconds` have passed.  Also: the same chain with the weight rows split
    over all host threads (a row split of the oracle's own calls), one pass of
    the 3B-class prefill at M = 512 and of the 70B-class layer at M = 128 on
    all threads, and the prefill on one thread over a bounded sample of rows."""
    import oracle
    from ternary_weight_linear_absmax_amd import inputs
    threads = _cpu_threads()
    prepared = []
    for i in range(len(inputs.DECODE_SHAPES)):
        _, w, x = inputs.decode(i, m=1)
        t, g = oracle.quantize_weights(w)
        prepared.append((x, t, g, oracle.pack2_pitch(w.shape[1]) * w.shape[0]))
    done_bytes, passes = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for x, t, g, nbytes in prepared:
            q, s, r = oracle.quantize_act(x)
            acc = oracle.matmul_i32(q, t)
            oracle.rescale(acc, s, g)
            done_bytes += nbytes
        passes += 1
    el = time.perf_counter() - t0
    out = {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle", "cpu_model": _cpu_model(), "host_threads_available": threads,
           "sample": f"{passes} passes over the 4 decode matrices (one layer, M=1) in "
                     f"{el:.1f} s; single-threaded scalar C"}
    log(f"cpu oracle decode, 1 thread: {out['value']} GB/s")

    # decode chain with the weight rows split over all threads
    done_bytes, passes = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds / 2:
        for x, t, g, nbytes in prepared:
            q, s, r = oracle.quantize_act(x)
            parts = _split_rows(lambda a, b: oracle.matmul_i32(q, t[a:b]), t.shape[0], threads)
            oracle.rescale(np.concatenate(parts, axis=1), s, g)
            done_bytes += nbytes
        passes += 1
    el = time.perf_counter() - t0
    out["all_cores"] = {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s",
                        "cores": threads,
                        "sample": f"{passes} passes over the 4 decode matrices, weight rows "
                                  f"split over {threads} threads, in {el:.1f} s"}
    log(f"cpu oracle decode, {threads} threads: {out['all_cores']['value']} GB/s")

    # prefill M=512 (one pass per shape on all threads; one thread on 32 rows)
    for si, (name, k, n) in enumerate(inputs.PREFILL_SHAPES):
        _, w, x = inputs.prefill(si)
        t, g = oracle.quantize_weights(w)
        m = x.shape[0]
        t0 = time.perf_counter()
        q, s, r = oracle.quantize_act(x)
        parts = _split_rows(lambda a, b: oracle.matmul_i32(q[a:b], t), m, threads)
        oracle.rescale(np.concatenate(parts, axis=0), s, g)
        el = time.perf_counter() - t0
        sub = 32
        t1 = time.perf_counter()
        q1, s1, _ = oracle.quantize_act(x[:sub])
        oracle.rescale(oracle.matmul_i32(q1, t), s1, g)
        el1 = time.perf_counter() - t1
        out[f"prefill_{name}_M512"] = {
            "TOPS": round(2.0 * m * n * k / el / 1e12, 5), "seconds": round(el, 2),
            "cores": threads,
            "one_thread_TOPS": round(2.0 * sub * n * k / el1 / 1e12, 5),
            "one_thread_sample": f"{sub} of {m} tokens in {el1:.2f} s"}
        log(f"cpu oracle prefill {name}: {el:.1f} s on {threads} threads")
    # 70B-class layer, M = 128 (one pass per shape on all threads)
    for si, (name, k, n) in enumerate(inputs.XL_SHAPES):
        _, w, x = inputs.xl(si, m=128)
        t, g = oracle.quantize_weights(w)
        del w
        m = x.shape[0]
        t0 = time.perf_counter()
        q, s, r = oracle.quantize_act(x)
        parts = _split_rows(lambda a, b: oracle.matmul_i32(q[a:b], t), m, threads)
        oracle.rescale(np.concatenate(parts, axis=0), s, g)
        el = time.perf_counter() - t0
        out[f"xl_{name}_M128"] = {"TOPS": round(2.0 * m * n * k / el / 1e12, 5),
                                  "GB/s_packed": round(n * oracle.pack2_pitch(k) / el / 1e9, 4),
                                  "seconds": round(el, 2), "cores": threads}
        log(f"cpu oracle xl {name} M=128: {el:.1f} s on {threads} threads")
        del t
    out.update(_cpu_stack(threads))
    return out


def _cpu_stack(threads, layers=2):
    """The oracle's 2B-class decoder layer at M = 64 (the layer-stack
    workload: RMSNorm + quantiser before every product, first-token GQA
    expansion, relu(gate)^2 * up, residual adds), every product's weight
    rows split over all threads; `layers` distinct layers timed, tokens/s
    extrapolated to the 30-layer step.  Weights are quantised before the
    timed region, as on the GPU."""
    import oracle
    from ternary_weight_linear_absmax_amd import inputs
    from ternary_weight_linear_absmax_amd import stack as st
    prepared = []
    for layer in range(layers):
        wl = inputs.stack_layer_weights(layer)
        prepared.append({name: oracle.quantize_weights(wl[name]) for name in st.MATRICES})
    x = oracle.bf16_to_f32(inputs.stack_input())
    m = x.shape[0]

    def product(qsr, tg):
        q, s, _ = qsr
        t, g = tg
        parts = _split_rows(lambda a, b: oracle.matmul_i32(q, t[a:b]), t.shape[0], threads)
        return oracle.rescale(np.concatenate(parts, axis=1), s, g).astype(np.float32)

    t0 = time.perf_counter()
    for lw in prepared:
        qkv = product(oracle.rmsnorm_quantize(x), lw["qkv"])
        v = qkv[:, st.V_COL:]
        o = product(oracle.rmsnorm_quantize(oracle.gqa_expand(v, st.HEADS, st.KV_HEADS)), lw["o"])
        x = oracle.add_f32(x, o)
        gu = product(oracle.rmsnorm_quantize(x), lw["up_gate"])
        d = product(oracle.rmsnorm_quantize(oracle.relu2_mul(gu[:, :st.FFN], gu[:, st.FFN:])),
                    lw["down"])
        x = oracle.add_f32(x, d)
    el = time.perf_counter() - t0
    per_layer = el / layers
    res = {"stack_2B_M64": {
        "tokens_per_s": round(m / (30 * per_layer), 2), "seconds_per_layer": round(per_layer, 3),
        "cores": threads,
        "sample": f"{layers} of the 30 layers at M = {m} in {el:.2f} s, extrapolated to 30"}}
    log(f"cpu oracle stack M={m}: {per_layer:.2f} s per layer on {threads} threads")
    return res


if __name__ == "__main__":
    main()
