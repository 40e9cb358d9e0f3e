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


def graph_time(fn, replays, warmup):
    """Capture fn() (a fixed sequence of launches) in one HIP graph and return
    the average ms per replay over `replays` back-to-back replays (HIP events
    on the replay stream).  Graph replay takes the Python and launch-queue
    overhead out of the timed region; every kernel still runs as launched."""
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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; run with --gpus 1 "
                          "(sharding over several GPUs is described, not implemented)"}))
        sys.exit(2)

    import torch
    from ternary_weight_linear_absmax_amd import bitlinear as bl
    from ternary_weight_linear_absmax_amd import inputs

    if args.calibrate_copy:
        calibrate_copy()
        return
    bl.load()
    dev_name = torch.cuda.get_device_name(0)
    log(f"device {dev_name}")

    # ---------------- headline: decode M=1, 30 layers -----------------------
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
    ms_step_eager = time_loop(step, max(2, args.steps // 10), 1)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"decode step {ms_step * 1e3:.1f} us (eager launches: {ms_step_eager * 1e3:.1f} us)"
        f" -> {value:.1f} GB/s")

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
                "algorithmic_bytes_per_launch": int(bytes_per_launch)}

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

    # ---------------- extra: 70B-class layer and prefill ------------------------
    extra = {}
    if not args.no_extra:
        extra = measure_extra(args)

    # ---------------- CPU oracle baseline ----------------------------------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager_launch": round(ms_step_eager, 4),
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
            "packed_bytes_per_step": step_bytes,
            "hbm_frac": round(value / HBM_PEAK_GBS, 4),
            "device": dev_name,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def measure_extra(args):
    """The other workloads, each timed as one captured graph of launches:
    the 70B-class layer (rotating 10 copies of each matrix, 587 MB, so the
    weights stream from HBM) at M = 1, 16, 128 and in base-3 at M = 1; the
    3B-class prefill GEMMs at M = 512."""
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
            ms = graph_time(fwd2, 20, 3) / copies_n
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
                ms3 = graph_time(fwd3, 20, 3) / copies_n
                gbs3 = p3.numel() / (ms3 * 1e-3) / 1e9
                extra[f"xl_{name}_M1_pack3"] = {
                    "K": k, "N": n, "M": 1, "us": round(ms3 * 1e3, 2), "GB/s": round(gbs3, 1),
                    "hbm_frac": round(gbs3 / HBM_PEAK_GBS, 4),
                    "trits_per_s": round(n * k / (ms3 * 1e-3), 1)}
                log(f"xl {name} M=1 pack3: {ms3 * 1e3:.1f} us {gbs3:.0f} GB/s")
        del c2, c3
        torch.cuda.empty_cache()
    # layer stack: 30 layers of the 2B-class decoder, M = 64 tokens at position 0
    extra.update(measure_stack(separate=not args.no_separate_stack))
    # prefill M=512 (packed weights 6.9 MB: they stay in the Infinity Cache)
    reps = 10
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
        ms = graph_time(fwd, 20, 3) / reps
        tops = 2.0 * m * n * k / (ms * 1e-3) / 1e12

        def full():
            for _ in range(reps):
                bl.quantize_act(xd)
                bl.forward(xq, scale, rowsum, packed, gamma, n, k, y=y)
        ms_full = graph_time(full, 20, 3) / reps
        extra[f"prefill_{name}_M512"] = {
            "K": k, "N": n, "M": m, "us": round(ms * 1e3, 2), "TOPS": round(tops, 2),
            "i8_frac": round(tops / I8_PEAK_TOPS, 4),
            "us_with_act_quant": round(ms_full * 1e3, 2),
            "TOPS_with_act_quant": round(2.0 * m * n * k / (ms_full * 1e-3) / 1e12, 2)}
        log(f"prefill {name}: {ms * 1e3:.1f} us {tops:.1f} TOPS")
    extra.update(measure_variants())
    extra.update(measure_backward())
    return extra


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
            ms = graph_time(bwd, 10, 2) / reps
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
    ms = graph_time(fwd, 20, 3) / len(copies)
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
    ms = graph_time(full4, 20, 3) / reps
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
        ms = graph_time(step, 20, 3)
        out[name] = {
            "layers": layers, "M": m, "us_per_step": round(ms * 1e3, 1),
            "tokens_per_s": round(m / (ms * 1e-3), 1), "packed_bytes": pb,
            "GB/s": round(pb / (ms * 1e-3) / 1e9, 1), "TOPS": round(ops / (ms * 1e-3) / 1e12, 2),
            "launches_per_step": per_layer * layers + 1}
        log(f"{name} {layers} layers M={m}: {ms * 1e3:.1f} us/step, "
            f"{m / (ms * 1e-3):.0f} tokens/s")
    del stack
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


def cpu_baseline(seconds):
    """The oracle, untuned, on this host: the decode workload's per-matrix chain
    (absmax quantisation, exact int32 product, rescale) at M = 1, repeated over
    the four shapes until `seconds` have passed."""
    import oracle
    from ternary_weight_linear_absmax_amd import inputs
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
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{passes} passes over the 4 decode matrices (one layer, M=1) in "
                      f"{el:.1f} s; single-threaded scalar C"}


if __name__ == "__main__":
    main()
