#!/usr/bin/env python3
"""Benchmark of the quantized-product hot path on one MI355X.

Headline (one JSON line on stdout):
  value   = decode weight GB/s: x bf16 [1,4096] times W [14336,4096] affine
            4-bit g64 with bf16 scales/biases (33,030,144 weight bytes per
            product), timed over exactly --steps products;
  prefill = TFLOP/s of x bf16 [2048,4096] times the same W (2*M*N*K flops),
            reported beside it with its own roofline.
Every other kernel of the path (quantize, dequantize, few-row, row-exact,
split-K, mixture-of-experts gather, the fp32 example) is timed too, under
"rows".

Timing: inputs are resident in HBM before the timed region; weight copies
rotate through >= 600 MB so the 256 MB last-level cache cannot serve them;
launches are captured in a HIP graph and replayed, bracketed by HIP events on
the launching stream and torch.cuda.synchronize() on both sides.

The CPU baseline times the plain CPU oracle (oracle/) on the same workload
on the host cores; it is a reported baseline, not a target.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "qmm weight GB/s at 1 row (decode); TFLOP/s at 2048 rows; 4-bit g64"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
ROTATE_BYTES = 600e6
PREROLL_CYCLES = 2_000_000     # spin before the timed region (clock ticks)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
CSRC = os.path.join(ROOT, "group_wise_affine_quantize_amd", "csrc")
KERNEL_SOURCES = {
    "decode_gemv": ["gemv.hip", "nq_device.h", "nq_internal.h"],
    "prefill": ["tiled.hip", "nq_device.h", "nq_internal.h"],
    "multirow_8bit": ["gemv_mfma.hip", "gemv.hip", "nq_device.h", "nq_internal.h"],
    "splitk": ["gemv.hip", "nq_device.h", "nq_internal.h"],
    "moe_gather": ["tiled.hip", "gemv.hip", "nq_device.h", "nq_internal.h"],
}


def source_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_record(kind):
    """The committed rocprofv3 figures of a workload's kernel (HBM bytes per
    launch from the counter passes, average duration from the kernel trace),
    if they were taken on the current kernel source; else {}."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError):
        return {}
    if not rec or rec.get("source_hash") != source_hash(kind):
        return {}
    return rec


def measured_traffic(kind):
    """HBM bytes per launch (None when the counters predate the source)."""
    return profile_record(kind).get("hbm_bytes_per_launch")


def trace_avg_us(kind):
    """The kernel trace's average duration in us (None when stale)."""
    return profile_record(kind).get("trace_avg_us")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="timed decode products")
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--row-steps", type=int, default=200, help="timed launches per other row")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU-oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch without HIP graphs")
    ap.add_argument("--only", choices=["decode", "prefill", "copy", "multirow_8bit", "splitk",
                                       "moe_gather"],
                    help="run one workload for a profiler and print its timing")
    return ap.parse_args()


class Timer:
    """Times `steps` launches of fn(i) on the current stream: captured into
    HIP graphs (or eager), HIP events around the timed region."""

    def __init__(self, torch, eager=False):
        self.torch = torch
        self.eager = eager

    def _graph(self, fn, start, count):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(start + i)
        return g

    def run(self, fn, steps, warmup, chunk=200):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(max(warmup, 1)):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        if not self.eager:
            chunk = max(1, min(chunk, steps))
            full, rest = divmod(steps, chunk)
            g_full = self._graph(fn, 0, chunk) if full else None
            g_rest = self._graph(fn, full * chunk, rest) if rest else None
            graphs = [g_full] * full + ([g_rest] if g_rest else [])
            for g in set(graphs):      # one untimed replay each
                g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # A spin kernel (about 1 ms) keeps the stream busy while the host
        # submits the timed work behind it, so the event window holds the
        # launches back to back and no host submission latency.
        torch.cuda._sleep(PREROLL_CYCLES)
        e0.record()
        if self.eager:
            for i in range(steps):
                fn(i)
        else:
            for g in graphs:
                g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3   # seconds


def prefill_only(args, B, synthetic, dev, q2, timer, log):
    """--only prefill: time the prefill product alone (for profiling)."""
    import torch
    x4 = dev(synthetic.generate("prefill")["x"])
    y4 = torch.empty((2048, 14336), dtype=torch.bfloat16, device="cuda")
    t = timer.run(lambda i: B.nq_qmm(x4, *q2, 64, 4, y=y4), args.prefill_steps, 3, chunk=10)
    log(f"prefill: {args.prefill_steps} launches, {t / args.prefill_steps * 1e6:.1f} us each")


def row_only(args, B, synthetic, dev, rotated, timer, log):
    """--only multirow_8bit | splitk | moe_gather: time that workload's batched
    (or grouped) product and its row-exact form, for a profiler."""
    import torch
    name = args.only
    wl = synthetic.WORKLOADS[name]
    d = synthetic.generate(name)
    q = B.nq_quantize(dev(d["w"]), wl.group_size, wl.bits)
    xs = dev(d["x"])
    cps = rotated(q)
    steps = args.row_steps
    if name == "moe_gather":
        ids = dev(d["ids"])
        rows, l, k = wl.x_shape
        e, n, _ = wl.w_shape
        y = torch.empty((rows, l, n), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(B.nq_gather_qmm_workspace_bytes(rows, l, k, e, n, wl.group_size, wl.bits,
                                                         torch.bfloat16, torch.bfloat16),
                         dtype=torch.uint8, device="cuda")
        entries = ((B.nq_gather_qmm, "grouped"), (B.nq_gather_qmm_row_exact, "row_exact"))
        for entry, tag in entries:
            t = timer.run(lambda i: entry(xs, *cps[i % len(cps)], wl.group_size, wl.bits, ids, y=y,
                                          workspace=ws), steps, 10)
            log(f"{name} {tag}: {steps} launches, {t / steps * 1e6:.3f} us each")
        return
    m, _ = wl.x_shape
    n = wl.w_shape[0]
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    for entry, tag in ((B.nq_qmm, "batched"), (B.nq_qmm_row_exact, "row_exact")):
        t = timer.run(lambda i: entry(xs, *cps[i % len(cps)], wl.group_size, wl.bits, y=y), steps, 10)
        log(f"{name} {tag}: {steps} launches, {t / steps * 1e6:.3f} us each")


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on a single GPU's share; see the design notes)", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from group_wise_affine_quantize_amd import _binding as B
    from group_wise_affine_quantize_amd import synthetic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    B.load_library()
    timer = Timer(torch, eager=args.eager)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        if a.dtype == np.uint32:
            return torch.from_numpy(a.view(np.int32)).cuda()
        return torch.from_numpy(a).cuda()

    def nbytes(*ts):
        return sum(t.numel() * t.element_size() for t in ts)

    def rotated(q, total=ROTATE_BYTES):
        per = nbytes(*q)
        copies = max(1, math.ceil(total / per))
        return [q] + [tuple(t.clone() for t in q) for _ in range(copies - 1)]

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    out = {"metric": METRIC}

    # ---------------------------------------------------------------- decode
    wl2 = synthetic.WORKLOADS["decode_gemv"]
    d2 = synthetic.generate("decode_gemv")
    w2 = dev(d2["w"])
    q2 = B.nq_quantize(w2, wl2.group_size, wl2.bits)
    torch.cuda.synchronize()
    weight_bytes = nbytes(*q2)
    assert weight_bytes == 33_030_144
    x2 = dev(d2["x"])
    y2 = torch.empty((1, 14336), dtype=torch.bfloat16, device="cuda")
    copies2 = rotated(q2)
    plan2 = B.nq_qmm_plan(1, 14336, 4096, 64, 4, torch.bfloat16, torch.bfloat16).as_dict()

    def decode(i):
        c, s, b = copies2[i % len(copies2)]
        B.nq_qmm(x2, c, s, b, 64, 4, y=y2)

    if args.only == "decode":
        t = timer.run(decode, args.steps, args.warmup)
        log(f"decode: {args.steps} launches, {t / args.steps * 1e6:.3f} us each")
        return
    if args.only == "copy":
        # a plain copy of known size, for scaling the HBM byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        t = timer.run(lambda i: dst.copy_(src), args.steps, args.warmup, chunk=20)
        log(f"copy: {args.steps} x {src.numel()} bytes, {t / args.steps * 1e6:.3f} us each")
        return

    if args.only == "prefill":
        return prefill_only(args, B, synthetic, dev, q2, timer, log)
    if args.only is not None:
        del copies2
        return row_only(args, B, synthetic, dev, rotated, timer, log)
    log("timing decode")
    t_dec = timer.run(decode, args.steps, args.warmup)
    # the graph replays must reproduce the eager result bit for bit
    y_eager = B.nq_qmm(x2, *copies2[(args.steps - 1) % len(copies2)], 64, 4)
    torch.cuda.synchronize()
    assert torch.equal(y_eager.view(torch.int16), y2.view(torch.int16))
    dec_launch_s = t_dec / args.steps
    dec_gbs = weight_bytes / dec_launch_s / 1e9
    out.update({
        "value": round(dec_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_dec / args.steps * 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_gemv: x bf16 [1,4096] . W[14336,4096]^T, affine 4-bit "
                               "group 64, bf16 scales/biases, y bf16 [1,14336]",
                   "weight_bytes_per_step": weight_bytes, "rotated_weight_copies": len(copies2),
                   "graph_replay": not args.eager, "plan": plan2},
    })
    traffic = measured_traffic("decode_gemv")
    out["roofline"] = {"bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                       "traffic": traffic, "kernel": "gemv_stream_kernel<bf16,2,14>",
                       "launch_us": round(dec_launch_s * 1e6, 3),
                       "trace_avg_us": trace_avg_us("decode_gemv")}
    del copies2

    # ---------------------------------------------------------------- prefill
    wl4 = synthetic.WORKLOADS["prefill"]
    x4 = dev(synthetic.generate("prefill")["x"])
    y4 = torch.empty((2048, 14336), dtype=torch.bfloat16, device="cuda")
    flops = 2 * 2048 * 14336 * 4096
    plan4 = B.nq_qmm_plan(2048, 14336, 4096, 64, 4, torch.bfloat16, torch.bfloat16).as_dict()

    def prefill(i):
        B.nq_qmm(x4, *q2, 64, 4, y=y4)

    log("timing prefill")
    t_pre = timer.run(prefill, args.prefill_steps, 3, chunk=10)
    pre_launch_s = t_pre / args.prefill_steps
    pre_tflops = flops / pre_launch_s / 1e12
    out["prefill"] = {
        "value": round(pre_tflops, 2), "unit": "TFLOP/s", "steps": args.prefill_steps,
        "ms_per_step": round(pre_launch_s * 1e3, 4),
        "config": {"workload": "prefill: x bf16 [2048,4096] . W[14336,4096]^T, affine 4-bit "
                               "group 64, fp32 accumulation, y bf16 [2048,14336]",
                   "flops_per_step": flops, "plan": plan4},
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("prefill"), "kernel": "tiled256_kernel<4,bf16>",
                     "launch_us": round(pre_launch_s * 1e6, 3), "trace_avg_us": trace_avg_us("prefill")},
    }

    # ---------------------------------------------------------------- other rows
    rows = {}
    if not args.no_rows:
        log("timing the other kernels")
        steps = args.row_steps

        def put(name, seconds, n, work, unit, extra=None):
            per = seconds / n
            rows[name] = {"us": round(per * 1e6, 3), unit: round(work / per / (1e9 if unit == "GB/s"
                                                                             else 1e12), 2)}
            if extra:
                rows[name].update(extra)

        # quantize: read W bf16, write codes, scales, biases
        w_copies = [w2] + [w2.clone() for _ in range(math.ceil(ROTATE_BYTES / nbytes(w2)) - 1)]
        qc = tuple(torch.empty_like(t) for t in q2)
        t = timer.run(lambda i: B.nq_quantize(w_copies[i % len(w_copies)], 64, 4, *qc), steps, 10)
        put("quantize", t, steps, nbytes(w2) + weight_bytes, "GB/s",
            {"workload": "W bf16 [14336,4096] -> 4-bit g64"})
        del w_copies
        wout = torch.empty((14336, 4096), dtype=torch.bfloat16, device="cuda")
        cps = rotated(q2)
        t = timer.run(lambda i: B.nq_dequantize(*cps[i % len(cps)], 64, 4, out=wout), steps, 10)
        put("dequantize", t, steps, nbytes(wout) + weight_bytes, "GB/s",
            {"workload": "4-bit g64 [14336,4096] -> bf16"})
        del cps

        for name in ("multirow_8bit", "splitk"):
            wl = synthetic.WORKLOADS[name]
            d = synthetic.generate(name)
            q = B.nq_quantize(dev(d["w"]), wl.group_size, wl.bits)
            xs = dev(d["x"])
            m, k = wl.x_shape
            n = wl.w_shape[0]
            ys = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
            cps = rotated(q)
            wb = nbytes(*q)
            for entry, tag in ((B.nq_qmm, "batched"), (B.nq_qmm_row_exact, "row_exact")):
                t = timer.run(lambda i: entry(xs, *cps[i % len(cps)], wl.group_size, wl.bits, y=ys),
                              steps, 10)
                put(f"{name}_{tag}", t, steps, wb, "GB/s",
                    {"workload": f"x bf16 [{m},{k}] . W[{n},{k}]^T {wl.bits}-bit g{wl.group_size}",
                     "plan": B.nq_qmm_plan(m, n, k, wl.group_size, wl.bits, torch.bfloat16,
                                           torch.bfloat16, tag == "row_exact").as_dict(),
                     "traffic": measured_traffic(name), "trace_avg_us": trace_avg_us(name)})
            del cps

        # the decode shape at the other code widths (3 and 6 straddle words)
        for bits in (2, 3, 6):
            qb = B.nq_quantize(w2, 64, bits)
            cps = rotated(qb)
            t = timer.run(lambda i: B.nq_qmm(x2, *cps[i % len(cps)], 64, bits, y=y2), steps, 10)
            put(f"decode_{bits}bit", t, steps, nbytes(*qb), "GB/s",
                {"workload": f"x bf16 [1,4096] . W[14336,4096]^T {bits}-bit g64"})
            del cps, qb

        # derivatives through the decode weights: dx = dy times the weights as
        # stored (1 row, and 2048 rows on the tiles), and the scale/bias
        # derivatives for one row
        cps = rotated(q2)
        dy1 = dev(synthetic.random_case(5, (1, 1), (1, 14336), 1.0, "f32", "bf16")[1])
        dx1 = torch.empty((1, 4096), dtype=torch.bfloat16, device="cuda")
        wsn = torch.empty(B.nq_qmm_notrans_workspace_bytes(1, 14336, 4096, 64, 4, torch.bfloat16),
                          dtype=torch.uint8, device="cuda")
        t = timer.run(lambda i: B.nq_qmm_notrans(dy1, *cps[i % len(cps)], 64, 4, y=dx1, workspace=wsn),
                      steps, 10)
        put("dx_decode", t, steps, weight_bytes, "GB/s",
            {"workload": "dx bf16 [1,4096] = dy [1,14336] . W[14336,4096] (weights as stored), 4-bit g64"})
        dsg = torch.empty((14336, 64), dtype=torch.float32, device="cuda")
        dbg = torch.empty_like(dsg)
        x1 = x2
        t = timer.run(lambda i: B.nq_qmm_grad_scales_biases(x1, dy1, cps[i % len(cps)][0], 64, 4,
                                                            dscales=dsg, dbiases=dbg), steps, 10)
        put("dscales_dbiases_decode", t, steps, nbytes(q2[0]) + 2 * nbytes(dsg), "GB/s",
            {"workload": "x [1,4096], dy [1,14336], codes of W[14336,4096] 4-bit g64 -> f32 [14336,64] x2"})
        del cps
        dyp = dev(synthetic.random_case(6, (1, 1), (2048, 14336), 1.0, "f32", "bf16")[1])
        dxp = torch.empty((2048, 4096), dtype=torch.bfloat16, device="cuda")
        tp = timer.run(lambda i: B.nq_qmm_notrans(dyp, *q2, 64, 4, y=dxp), max(2, steps // 20), 2)
        put("dx_prefill", tp, max(2, steps // 20), 2 * 2048 * 14336 * 4096, "TFLOP/s",
            {"workload": "dx bf16 [2048,4096] = dy [2048,14336] . W[14336,4096] (128-row tiles)"})
        del dyp, dxp

        wl = synthetic.WORKLOADS["moe_gather"]
        d = synthetic.generate("moe_gather")
        q = B.nq_quantize(dev(d["w"]), wl.group_size, wl.bits)
        xs, ids = dev(d["x"]), dev(d["ids"])
        yg = torch.empty((512, 1, 1408), dtype=torch.bfloat16, device="cuda")
        wsg = torch.empty(B.nq_gather_qmm_workspace_bytes(512, 1, 2048, 32, 1408, 64, 4,
                                                          torch.bfloat16, torch.bfloat16),
                          dtype=torch.uint8, device="cuda")
        cps = rotated(q)
        for entry, tag in ((B.nq_gather_qmm, "moe_gather"),
                           (B.nq_gather_qmm_row_exact, "moe_gather_row_exact")):
            t = timer.run(lambda i: entry(xs, *cps[i % len(cps)], 64, 4, ids, y=yg, workspace=wsg),
                          steps, 10)
            extra = {"workload": "x bf16 [512,1,2048], 32 experts W[1408,2048] 4-bit g64, "
                                 "unsorted ids (grouped by expert on the device)",
                     "tflops": round(2 * 512 * 1408 * 2048 / (t / steps) / 1e12, 3)}
            if tag == "moe_gather":
                extra.update({"traffic": measured_traffic("moe_gather"),
                              "trace_avg_us": trace_avg_us("moe_gather")})
            put(tag, t, steps, nbytes(*q), "GB/s", extra)
        del cps

        wl = synthetic.WORKLOADS["affine_f32_256x512"]
        d = synthetic.generate("affine_f32_256x512")
        q = B.nq_quantize(dev(d["w"]), 64, 4)
        xs = dev(d["x"])
        y1 = torch.empty((4, 256), dtype=torch.float32, device="cuda")
        t = timer.run(lambda i: B.nq_qmm(xs, *q, 64, 4, y=y1), steps, 10)
        put("affine_f32_256x512", t, steps, nbytes(*q), "GB/s",
            {"workload": "x f32 [4,512] . W[256,512]^T 4-bit g64 f32 scales (launch-bound)"})

        # floating-point modes (uniformly random codes; moderate scale codes)
        fp_scales = {"mxfp4": (120, 134), "mxfp8": (120, 134), "nvfp4": (0x20, 0x50)}

        def fp_weights(mode, lead, k, seed):
            _, bits, gs = B.FP_MODES[mode]
            wds, scs = synthetic.random_fp_matrix(seed, lead, k, bits, gs, fp_scales[mode],
                                                  finite_bytes=True)
            return dev(wds), torch.from_numpy(scs).cuda()

        qf = tuple(torch.empty_like(t) for t in B.nq_fp_quantize(w2, "mxfp4"))
        w_copies = [w2] + [w2.clone() for _ in range(math.ceil(ROTATE_BYTES / nbytes(w2)) - 1)]
        t = timer.run(lambda i: B.nq_fp_quantize(w_copies[i % len(w_copies)], "mxfp4", *qf), steps, 10)
        put("fp_quantize_mxfp4", t, steps, nbytes(w2) + nbytes(*qf), "GB/s",
            {"workload": "W bf16 [14336,4096] -> MXFP4 codes and E8M0 scales"})
        del w_copies
        for mode in ("mxfp4", "mxfp8", "nvfp4"):
            qm = fp_weights(mode, (14336,), 4096, 31)
            cps = rotated(qm)
            t = timer.run(lambda i: B.nq_fp_qmm(x2, *cps[i % len(cps)], mode, y=y2), steps, 10)
            put(f"fp_decode_{mode}", t, steps, nbytes(*qm), "GB/s",
                {"workload": f"x bf16 [1,4096] . W[14336,4096]^T {mode}"})
            if mode == "mxfp4":
                # the derivative for the activations through these weights (as stored)
                dyf = dev(synthetic.random_case(7, (1, 1), (1, 14336), 1.0, "f32", "bf16")[1])
                dxf = torch.empty((1, 4096), dtype=torch.bfloat16, device="cuda")
                wsf = torch.empty(B.nq_fp_qmm_notrans_workspace_bytes(1, 14336, 4096, mode, torch.bfloat16),
                                  dtype=torch.uint8, device="cuda")
                t = timer.run(lambda i: B.nq_fp_qmm_notrans(dyf, *cps[i % len(cps)], mode, y=dxf, workspace=wsf),
                              steps, 10)
                put("fp_dx_decode_mxfp4", t, steps, nbytes(*qm), "GB/s",
                    {"workload": "dx bf16 [1,4096] = dy [1,14336] . W[14336,4096] mxfp4 (weights as stored)"})
                dyp = dev(synthetic.random_case(8, (1, 1), (2048, 14336), 1.0, "f32", "bf16")[1])
                dxp = torch.empty((2048, 4096), dtype=torch.bfloat16, device="cuda")
                tp = timer.run(lambda i: B.nq_fp_qmm_notrans(dyp, *qm, mode, y=dxp), max(2, steps // 20), 2)
                put("fp_dx_prefill_mxfp4", tp, max(2, steps // 20), 2 * 2048 * 14336 * 4096, "TFLOP/s",
                    {"workload": "dx bf16 [2048,4096] = dy [2048,14336] . W[14336,4096] mxfp4 (128x128 tiles)"})
                del dyp, dxp
                t = timer.run(lambda i: B.nq_fp_dequantize(*cps[i % len(cps)], mode, out=wout), steps, 10)
                put("fp_dequantize_mxfp4", t, steps, nbytes(wout) + nbytes(*qm), "GB/s",
                    {"workload": "MXFP4 [14336,4096] -> bf16"})
                yp = torch.empty((2048, 14336), dtype=torch.bfloat16, device="cuda")
                tp = timer.run(lambda i: B.nq_fp_qmm(x4, *qm, mode, y=yp), max(2, steps // 20), 2)
                put("fp_prefill_mxfp4", tp, max(2, steps // 20), 2 * 2048 * 14336 * 4096, "TFLOP/s",
                    {"workload": "x bf16 [2048,4096] . W[14336,4096]^T mxfp4 (128x128 tiles)"})
                del yp
            del cps, qm
        del wout
        cg, sg = fp_weights("nvfp4", (32, 1408), 2048, 32)
        gsc = torch.rand(32, dtype=torch.float32, device="cuda") + 0.5
        xg = dev(synthetic.generate("moe_gather")["x"])
        idg = dev(synthetic.generate("moe_gather")["ids"])
        wsf = torch.empty(B.nq_fp_gather_qmm_workspace_bytes(512, 1, 2048, 32, 1408), dtype=torch.uint8,
                          device="cuda")
        for tag, rx in (("fp_gather_nvfp4", False), ("fp_gather_nvfp4_row_exact", True)):
            t = timer.run(lambda i: B.nq_fp_gather_qmm(xg, cg, sg, "nvfp4", idg, global_scales=gsc,
                                                       row_exact=rx, y=yg, workspace=wsf), steps, 10)
            put(tag, t, steps, nbytes(cg, sg), "GB/s",
                {"workload": "x bf16 [512,1,2048], 32 NVFP4 experts W[1408,2048] with global scales, "
                             "unsorted ids grouped by expert on the device" +
                             (" (row-exact matrix-vector route)" if rx else " (matrix-core route)"),
                 "tflops": round(2 * 512 * 1408 * 2048 / (t / steps) / 1e12, 3)})
    out["rows"] = rows

    # ---------------------------------------------------------------- measured ceilings
    # Context only (no product code): what this GPU's library paths reach on
    # the same data sizes -- a 1 GiB device copy (HBM read + write), a read
    # of 1 GiB (torch's max over int64 elements: one read stream, a few
    # bytes written) and a dense bf16 matmul (hipBLASLt through torch) of the
    # prefill shape with the weights already dequantized.
    if not args.no_rows:
        log("timing the context ceilings")
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        t = timer.run(lambda i: dst.copy_(src), 20, 3, chunk=10)
        copy_gbs = 2 * src.numel() / (t / 20) / 1e9
        del dst
        # eager launches: a multi-block reduction records memsets, kept out of
        # graphs; max over int64 is the fastest of torch's reductions here
        src64 = src.view(torch.int64)
        t = Timer(torch, eager=True).run(lambda i: src64.max(), 20, 3, chunk=10)
        read_gbs = src.numel() / (t / 20) / 1e9
        del src, src64
        w_hat = B.nq_dequantize(*q2, 64, 4)
        yd = torch.empty((2048, 14336), dtype=torch.bfloat16, device="cuda")
        t = timer.run(lambda i: torch.matmul(x4, w_hat.t(), out=yd), 20, 3, chunk=10)
        out["context"] = {
            "hbm_copy_1GiB_GBs": round(copy_gbs, 1),
            "hbm_read_1GiB_GBs": round(read_gbs, 1),
            "dense_bf16_matmul_prefill_shape_TFLOPs": round(flops / (t / 20) / 1e12, 1),
            "note": "torch copy_, max and matmul (hipBLASLt) on the same GPU; not the product path",
        }
        del w_hat, yd

    # ---------------------------------------------------------------- CPU oracle
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        import oracle as O
        c_np = q2[0].cpu().numpy().view(np.uint32)
        s_np = q2[1].cpu().view(torch.int16).numpy().view(np.uint16)
        b_np = q2[2].cpu().view(torch.int16).numpy().view(np.uint16)
        times = []
        t_end = time.perf_counter() + args.cpu_seconds
        while len(times) < 3 or (time.perf_counter() < t_end and len(times) < 200):
            t0 = time.perf_counter()
            O.qmm_f64(d2["x"], c_np, s_np, b_np, 64, 4)
            times.append(time.perf_counter() - t0)
        t_cpu = statistics.median(times)
        out["cpu_baseline"] = {
            "value": round(weight_bytes / t_cpu / 1e9, 4), "unit": "GB/s",
            "cores": O.threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"the whole decode workload (x [1,4096] . W[14336,4096]^T, fp64 "
                      f"accumulation), median of {len(times)} runs",
        }
        x4h = synthetic.generate("prefill")["x"][:8]
        t0 = time.perf_counter()
        O.qmm_f64(x4h, c_np, s_np, b_np, 64, 4)
        t_pre_cpu = time.perf_counter() - t0
        out["prefill"]["cpu_baseline"] = {
            "value": round(2 * 8 * 14336 * 4096 / t_pre_cpu / 1e12, 6), "unit": "TFLOP/s",
            "cores": O.threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "8 of the 2048 prefill rows against all of W (1 run)"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
