"""Benchmark: forward convolution TFLOPS and roofline fraction on one MI355X.

A step is one conv2d_fwd call -- every step of the path (the lowering
structure build, the MFMA main loop and its fused epilogue, and any split-K
finish) -- over one batch of seeded synthetic input that is already resident
in HBM.  Before each timed step the 256 MB last-level cache (MALL) is
overwritten, outside the timed interval, so the input really comes from HBM.
Each step is bracketed by HIP events on the stream the library launches on;
ms_per_step is their mean.

Headline: the 3x3 stride-1 pad-1 layer N=32, C_in=64, 56x56, C_out=128 in
bf16, NCHW, algo auto -- the verification layer of "Unifying Convolutions and
GEMM", section 5.  The JSON line also carries a per-layer table over every
layer shape (TFLOPS, roofline fraction, workspace vs im2col bytes), the
dominant kernel's roofline entry (its duration measured with HIP events on
the main loop alone), and the fp64 oracle's throughput on this host's cores
over a bounded sample (a baseline only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers all|headline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "conv fwd TFLOPS & fraction of MFMA peak per layer; workspace bytes"
PEAK = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}  # MI355X dense MFMA, TFLOP/s
HBM_PEAK = 8000.0  # GB/s
ESIZE = {"bf16": 2, "fp16": 2, "fp32": 4}


def layer_geometry(L):
    import convolution_lowering_amd as cl
    Ho, Wo = cl.output_size(L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation)
    return Ho, Wo


def layer_flops(L, Ho, Wo):
    return 2.0 * L.N * L.Co * Ho * Wo * L.C * L.KH * L.KW


def algorithmic_bytes(L, Ho, Wo, dtype):
    """Each tensor moved once: |x| + |w| + |bias| + |y|."""
    e = ESIZE[dtype]
    return e * (L.N * L.C * L.H * L.W + L.Co * L.C * L.KH * L.KW + L.Co + L.N * L.Co * Ho * Wo)


def roofline(flops, nbytes, seconds, dtype):
    intensity = flops / nbytes
    ridge = PEAK[dtype] * 1e12 / (HBM_PEAK * 1e9)
    if intensity >= ridge:
        ach = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": PEAK[dtype], "unit": "TFLOP/s", "frac": ach / PEAK[dtype]}
    ach = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK, "unit": "GB/s", "frac": ach / HBM_PEAK}


class Flusher:
    """Overwrites 512 MB so the 256 MB MALL holds none of the next step's inputs."""

    def __init__(self):
        import torch
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        self.i = 0

    def __call__(self):
        self.i = (self.i + 1) & 0xFF
        self.buf.fill_(self.i)


def time_steps(fn, steps, warmup, flush, stamp_main_loop=False):
    """Mean and minimum milliseconds of fn() over `steps` calls, each between
    HIP events on torch's current stream (the stream the library launches
    on).  With stamp_main_loop, also the mean and minimum duration of the
    main-loop kernel inside each timed call, from events that kernel stamps
    itself at its start and end (conv2d_time_next_main_loop)."""
    import torch
    import convolution_lowering_amd as cl
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    kev = []
    if stamp_main_loop:
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in kev:  # create the device events before the kernel stamps them
            a.record()
            b.record()
        torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        if flush:
            flush()
        if kev:
            cl.time_next_main_loop(*kev[i])
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in ev]
    out = (sum(times) / len(times), min(times))
    if kev:
        kt = [a.elapsed_time(b) for a, b in kev]
        out += (sum(kt) / len(kt), min(kt))
    return out


def bench_layer(L, dtype, layout, algo, steps, warmup, flush, stamp_main_loop=False):
    import torch
    import convolution_lowering_amd as cl
    from convolution_lowering_amd.workloads import make_inputs
    x, w, b = make_inputs(L, dtype, layout)
    x, w, b = x.cuda(), w.cuda(), b.cuda()
    Ho, Wo = layer_geometry(L)
    shape = (L.N, L.Co, Ho, Wo) if layout == "NCHW" else (L.N, Ho, Wo, L.Co)
    y = torch.empty(shape, dtype=x.dtype, device="cuda")
    ws_bytes = cl.workspace_size(L.N, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation, layout, dtype, algo)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        cl.conv2d_fwd(x, w, b, L.stride, L.pad, L.dilation, layout, algo, out=y, workspace=ws[:ws_bytes])

    ms, ms_min = time_steps(step, steps, warmup, flush)
    if stamp_main_loop:
        # A second pass of the same steps in which the main-loop kernel
        # stamps its own start and end (a launch with stamps takes a few
        # microseconds longer to dispatch, so the step time above comes from
        # the pass without them).
        t = time_steps(step, steps, 0, flush, True)
    flops = layer_flops(L, Ho, Wo)
    nbytes = algorithmic_bytes(L, Ho, Wo, dtype)
    im2col = cl.im2col_bytes(L.N, L.C, L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation, dtype)
    row = {"layer": L.name, "shape": L.note, "dtype": dtype, "layout": layout, "algo": algo,
           "ms": ms, "ms_min": ms_min, "tflops": flops / ms / 1e9, "gbps": nbytes / ms / 1e6,
           "workspace_bytes": ws_bytes, "im2col_bytes": im2col,
           "workspace_over_im2col": ws_bytes / im2col}
    row["roofline"] = roofline(flops, nbytes, ms / 1e3, dtype)
    if stamp_main_loop:
        row["main_loop_ms"], row["main_loop_ms_min"] = t[2], t[3]
    del x, w, b, y, ws
    return row


# The sources the headline main loop (igemm_rowwin_kernel, its epilogue and
# its launch) and the host planner that picks it are built from; a change to
# any of them invalidates the committed HBM counters of that kernel.
HEADLINE_SOURCES = ("conv_api.cpp", "conv_internal.h", "igemm_dma.h", "igemm_dual.h", "igemm_impl.h",
                    "igemm_inst.hip", "igemm_rowwin.h")


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "convolution_lowering_amd", "csrc")
    for f in HEADLINE_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    ent = rec.get(workload)
    if not ent or ent.get("source_digest") != kernel_source_digest():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(L, dtype, layout, budget_s=10.0):
    """The fp64 oracle (untuned) on the headline layer's whole batch, repeated
    until about budget_s seconds have passed (at least once); its mean rate."""
    import oracle
    from convolution_lowering_amd.workloads import make_inputs
    Ho, Wo = layer_geometry(L)
    lay = oracle.NCHW if layout == "NCHW" else oracle.NHWC
    x, w, b = make_inputs(L, dtype, layout)
    reps, t = 0, 0.0
    while reps == 0 or t < budget_s:
        t0 = time.perf_counter()
        oracle.conv2d(x, w, b, L.stride, L.pad, L.dilation, lay, want_norm=False)
        t += time.perf_counter() - t0
        reps += 1
    flops = layer_flops(L, Ho, Wo) * reps
    return {"value": flops / t / 1e12, "unit": "TFLOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole batch ({L.N} images) of the headline layer, full fp64 output, "
                      f"{reps} repetition(s), {t:.1f} s"}


def calibration_copy(nbytes=256 << 20):
    """One plain device copy of known size, so HBM byte counters read in the
    same profiled run can be scaled (bytes read and written = nbytes each)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(3)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", choices=["all", "headline"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one 256 MiB device copy (scale reference for HBM byte counters)")
    ap.add_argument("--only", metavar="LAYER:LAYOUT[:DTYPE]",
                    help="time only this layer (algo auto, dtype bf16 unless given) and print its row; "
                         "for profiling one layer's kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path (each GPU would run its own "
              "share of the batch independently; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import convolution_lowering_amd as cl
    from convolution_lowering_amd.workloads import LAYERS
    cl.lib()
    torch.cuda.init()
    flush = Flusher()
    # Bring the GPU out of its idle clock state before anything is timed:
    # about half a second of memory traffic (no step is run here).
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        for _ in range(20):
            flush()
        torch.cuda.synchronize()

    if args.only:
        parts = args.only.split(":")
        L = LAYERS[parts[0]]
        row = bench_layer(L, parts[2] if len(parts) > 2 else "bf16", parts[1], "auto", args.steps, args.warmup, flush)
        if args.calibration_copy:
            calibration_copy()
        print(json.dumps(row))
        return

    H = LAYERS["C2"]
    head_dtype, head_layout, head_algo = "bf16", "NCHW", "auto"
    head = bench_layer(H, head_dtype, head_layout, head_algo, args.steps, args.warmup, flush, stamp_main_loop=True)
    print(f"# headline {H.name} {head_dtype} {head_layout} {head_algo}: {head['ms']:.4f} ms "
          f"{head['tflops']:.1f} TFLOPS", file=sys.stderr, flush=True)
    try:  # the graphics clock right after the headline steps (amd-smi through torch)
        clock_mhz = float(torch.cuda.clock_rate())
    except Exception:
        clock_mhz = None

    # Roofline entry of the dominant kernel, the main loop with its fused
    # epilogue: its own duration inside the timed headline steps.
    ml_ms = head["main_loop_ms"]
    Ho, Wo = layer_geometry(H)
    flops = layer_flops(H, Ho, Wo)
    nbytes = algorithmic_bytes(H, Ho, Wo, head_dtype)
    rl = roofline(flops, nbytes, ml_ms / 1e3, head_dtype)
    rl["traffic"] = measured_traffic("C2-bf16-NCHW-main-loop")
    rl["kernel"] = ("igemm_rowwin_kernel (MFMA implicit-GEMM main loop over window rows staged in LDS + fused "
                    "bias epilogue)")
    rl["ms"] = ml_ms
    rl["timing"] = ("mean of the kernel's own start/end stamps (hipExtLaunchKernel events) over a second "
                    "timed pass of the headline steps")
    rl["per_launch_flops"] = flops
    rl["per_launch_algorithmic_bytes"] = nbytes

    rows = []
    if args.layers == "all":
        for name, L in LAYERS.items():
            # fp16 on the verification layer too (the second 16-bit type)
            for dtype in (L.dtypes + ("fp16",) if name == "C2" else L.dtypes):
                for layout in ("NCHW", "NHWC"):
                    # every layer also through the two baselines: the
                    # materialised im2col the lowering avoids, and direct
                    # convolution on the vector ALUs
                    algos = ["auto", "im2col", "direct", "im2win_lds"]
                    if name == "C2":
                        algos = ["auto", "indirect", "im2win", "im2col", "direct", "im2win_lds"]
                    for algo in algos:
                        try:
                            r = bench_layer(L, dtype, layout, algo, max(3, args.steps // 4), 2, flush)
                        except cl.ConvLowerError as e:
                            if algo == "im2win_lds" and e.code == 2:
                                continue  # shape outside the window-rows-in-LDS loop
                            r = {"layer": name, "dtype": dtype, "layout": layout, "algo": algo, "error": str(e)}
                        except Exception as e:  # report, keep going
                            r = {"layer": name, "dtype": dtype, "layout": layout, "algo": algo, "error": str(e)}
                        rows.append(r)
                        print(f"# {name} {dtype} {layout} {algo}: "
                              f"{r.get('ms', float('nan')):.4f} ms {r.get('tflops', float('nan')):.1f} TFLOPS "
                              f"{r.get('roofline', {}).get('bound', '?')} "
                              f"frac {r.get('roofline', {}).get('frac', float('nan')):.3f}", file=sys.stderr, flush=True)
                        torch.cuda.empty_cache()

    # Ablation of the main loop's techniques: every variant forced on a few
    # layers (same whole-call timing).
    ablation = []
    if args.layers == "all":
        for name, dtype, layout in (("C2", "bf16", "NCHW"), ("C2", "bf16", "NHWC"), ("C3c", "bf16", "NHWC"),
                                    ("C4d", "bf16", "NHWC")):
            L = LAYERS[name]
            for variant in cl.MAIN_LOOPS:
                cl.force_main_loop(variant)
                try:
                    r = bench_layer(L, dtype, layout, "auto", max(3, args.steps // 4), 2, flush)
                    ablation.append({"layer": name, "dtype": dtype, "layout": layout, "main_loop": variant,
                                     "ms": r["ms"], "tflops": r["tflops"]})
                    print(f"# ablation {name} {dtype} {layout} {variant}: {r['ms']:.4f} ms {r['tflops']:.1f} TFLOPS",
                          file=sys.stderr, flush=True)
                except cl.ConvLowerError as e:
                    ablation.append({"layer": name, "dtype": dtype, "layout": layout, "main_loop": variant,
                                     "error": str(e)})
                finally:
                    cl.force_main_loop("auto")
                torch.cuda.empty_cache()

    if args.calibration_copy:
        calibration_copy()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(H, head_dtype, head_layout)

    line = {
        "metric": METRIC, "value": head["tflops"], "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": head_dtype,
        "data": "synthetic (seeded torch CPU generator; x, w, bias ~ N(0,1)), MALL flushed before each step",
        "config": {"workload": "conv2d fwd 3x3 s1 p1 N=32 C_in=64 56x56 C_out=128 (C2)", "layout": head_layout,
                   "algo": head_algo, "global_batch": H.N,
                   "workspace_bytes": head["workspace_bytes"], "im2col_bytes": head["im2col_bytes"]},
        "roofline": rl,
        "gpu_clock_mhz_after_headline": clock_mhz,
        "cpu_baseline": cpu,
        "layers": rows,
        "ablation": ablation,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
