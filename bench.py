"""Benchmark: forward convolution TFLOPS and roofline fraction on one MI355X.

Workload of the headline: the VGG-16-shaped set of 3x3 stride-1 pad-1
layers at N=128 in bf16, NCHW (C_in -> C_out at H=W: 3->64@224, 64->128@112,
128->256@56, 256->512@28, 512->512@14), each with its own seeded synthetic
x ~ U[-1,1], Kaiming-normal w and N(0,1) bias, already resident in HBM.  A
step is one conv2d_fwd call per layer of the set, every step of the path
inside it (any lowering launch, the MFMA main loop with its fused epilogue,
any split-K finish).  Before each timed step, outside the timed interval,
512 MB are overwritten and then another 512 MB buffer is read, so the 256 MB
last-level cache (MALL) holds none of the step's inputs (they come from HBM)
and no lines still to be written back.  Each step, and each layer inside
it, is bracketed by HIP events on the stream the library launches on.  The
warm-up steps are preceded by half a second of untimed steps, so that the
shader clock has settled before anything is timed.

The last line of stdout is one compact JSON object: the set's TFLOPS, the
per-layer times, the roofline entry of the dominant kernel (the main loop of
the 64->128@112 layer, timed by events the kernel stamps itself at its start
and end), and the fp64 oracle's rate on this host's cores over a bounded
sample of the same workload (a baseline only).  `--layers all` also times
every layer shape of the shape table under every algorithm, and the main-loop
ablation, and writes those rows to the file `--rows-out` names (they also go
to stderr, one per line), never to the last line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers headline|all] [--rows-out FILE]
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
PEAK = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3, "fp8": 5000.0}  # MI355X dense MFMA, TFLOP/s
HBM_PEAK = 8000.0  # GB/s
ESIZE = {"bf16": 2, "fp16": 2, "fp32": 4, "fp8": 1}
OUT_ESIZE = {"bf16": 2, "fp16": 2, "fp32": 4, "fp8": 2}  # y and bias (bf16 for fp8 inputs)

HEAD_SET = ("C4a", "C4b", "C4c", "C4d", "C4e")
HEAD_DTYPE, HEAD_LAYOUT, HEAD_ALGO = "bf16", "NCHW", "auto"
HEAD_DOMINANT = "C4b"  # the layer whose main loop takes the largest share of a step
HEAD_WORKLOAD = ("VGG-16-shaped 3x3 s1 p1 layer set, bf16, N=128, NCHW: 3->64@224, 64->128@112, "
                 "128->256@56, 256->512@28, 512->512@14")
# Images of each layer of the set the CPU baseline runs the oracle on.
CPU_SAMPLE_IMAGES = 16


def layer_geometry(L):
    import convolution_lowering_amd as cl
    return cl.output_size(L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation)


def layer_flops(L, Ho, Wo, n=None):
    return 2.0 * (L.N if n is None else n) * L.Co * Ho * Wo * L.C * L.KH * L.KW


def algorithmic_bytes(L, Ho, Wo, dtype):
    """Each tensor moved once: |x| + |w| + |bias| + |y|."""
    e, eo = ESIZE[dtype], OUT_ESIZE[dtype]
    return e * (L.N * L.C * L.H * L.W + L.Co * L.C * L.KH * L.KW) + eo * (L.Co + L.N * L.Co * Ho * Wo)


def roofline(flops, nbytes, seconds, dtype):
    intensity = flops / nbytes
    ridge = PEAK[dtype] * 1e12 / (HBM_PEAK * 1e9)
    if intensity >= ridge:
        ach = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": PEAK[dtype], "unit": "TFLOP/s", "frac": ach / PEAK[dtype]}
    ach = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK, "unit": "GB/s", "frac": ach / HBM_PEAK}


class Flusher:
    """Empties the 256 MB MALL of the next step's inputs and of dirty lines.

    Overwriting 512 MB evicts everything, but leaves the MALL full of written
    lines; the first kernel timed after it would then pay for writing them
    back (same box: the 1x1 256->64 @56 layer 48 -> 31 us, the 3->64 @224
    stem 190 -> 156 us once a read follows the fill).  So a second 512 MB
    buffer, which no layer touches, is read afterwards: its clean lines
    replace the written ones, whose write-back happens inside the flush."""

    def __init__(self):
        import torch
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        self.rbuf = torch.zeros(64 << 20, dtype=torch.int64, device="cuda")  # 512 MB
        self.i = 0

    def __call__(self):
        self.i = (self.i + 1) & 0xFF
        self.buf.fill_(self.i)
        self.rbuf.amax()


class Prepared:
    """One layer's device tensors (inputs, output, workspace) and its call."""

    def __init__(self, L, dtype, layout, algo, keep_host_images=0):
        import torch
        import convolution_lowering_amd as cl
        from convolution_lowering_amd.workloads import make_inputs
        x, w, b = make_inputs(L, dtype, layout)
        # The first images of the batch, kept on the host for the oracle.
        self.host = (x[:keep_host_images].clone(), w.clone(), b.clone()) if keep_host_images else None
        self.L, self.dtype, self.layout, self.algo = L, dtype, layout, algo
        self.x, self.w, self.b = x.cuda(), w.cuda(), b.cuda()
        del x, w, b
        Ho, Wo = layer_geometry(L)
        self.Ho, self.Wo = Ho, Wo
        shape = (L.N, L.Co, Ho, Wo) if layout == "NCHW" else (L.N, Ho, Wo, L.Co)
        self.y = torch.empty(shape, dtype=self.b.dtype, device="cuda")
        self.ws_bytes = cl.workspace_size(L.N, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation,
                                          layout, dtype, algo)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device="cuda")
        self.im2col = cl.im2col_bytes(L.N, L.C, L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation, dtype)
        self.flops = layer_flops(L, Ho, Wo)
        self.nbytes = algorithmic_bytes(L, Ho, Wo, dtype)

    def __call__(self):
        import convolution_lowering_amd as cl
        L = self.L
        cl.conv2d_fwd(self.x, self.w, self.b, L.stride, L.pad, L.dilation, self.layout, self.algo, out=self.y,
                      workspace=self.ws[:self.ws_bytes])


def time_set(layers, steps, warmup, flush, stamp=None):
    """Times `steps` steps, each one call per prepared layer in order, with
    events on torch's current stream (the stream the library launches on)
    before the step, after every layer and after the step.  Returns the mean
    and minimum step time and the mean time of each layer, in ms.

    stamp = index of a layer: in every timed step that layer's main-loop
    kernel stamps two events itself, at its own start and end
    (conv2d_time_next_main_loop); the mean and minimum of that duration are
    returned as well."""
    import torch
    import convolution_lowering_amd as cl
    for _ in range(warmup):
        for p in layers:
            p()
    torch.cuda.synchronize()
    n = len(layers)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    kev = []
    if stamp is not None:
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in kev:  # create the device events before the kernel stamps them
            a.record()
            b.record()
        torch.cuda.synchronize()
    for i in range(steps):
        if flush:
            flush()
        ev[i][0].record()
        for j, p in enumerate(layers):
            if stamp == j:
                cl.time_next_main_loop(*kev[i])
            p()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    step = [e[0].elapsed_time(e[n]) for e in ev]
    per_layer = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / steps for j in range(n)]
    out = {"ms": sum(step) / steps, "ms_min": min(step), "layer_ms": per_layer}
    if kev:
        kt = [a.elapsed_time(b) for a, b in kev]
        out["kernel_ms"], out["kernel_ms_min"] = sum(kt) / steps, min(kt)
    return out


def layer_row(p, ms, ms_min=None):
    row = {"layer": p.L.name, "shape": p.L.note, "dtype": p.dtype, "layout": p.layout, "algo": p.algo,
           "ms": ms, "tflops": p.flops / ms / 1e9, "workspace_bytes": p.ws_bytes, "im2col_bytes": p.im2col,
           "roofline": roofline(p.flops, p.nbytes, ms / 1e3, p.dtype)}
    if ms_min is not None:
        row["ms_min"] = ms_min
    return row


def bench_layer(L, dtype, layout, algo, steps, warmup, flush):
    """One layer alone (the sweep and the ablation): its row."""
    import torch
    p = Prepared(L, dtype, layout, algo)
    t = time_set([p], steps, warmup, flush)
    row = layer_row(p, t["ms"], t["ms_min"])
    del p
    torch.cuda.empty_cache()
    return row


# The sources the dominant kernel (the window-row main loop, its epilogue and
# its launch) and the host planner that picks it are built from; a change to
# any of them invalidates the committed HBM counters of that kernel.
HEADLINE_SOURCES = ("conv_api.cpp", "conv_internal.h", "igemm_dma.h", "igemm_dual.h", "igemm_impl.h",
                    "igemm_inst.hip", "igemm_rowwin.h")
TRAFFIC_KEY = "C4b-bf16-NCHW-main-loop"


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "convolution_lowering_amd", "csrc")
    for f in HEADLINE_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    ent = rec.get(key)
    if not ent or ent.get("source_digest") != kernel_source_digest():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(prepared, layout, budget_s=10.0):
    """The fp64 oracle (untuned) on the first CPU_SAMPLE_IMAGES images of every
    layer of the set, the same values the GPU step multiplies, repeated until
    about budget_s seconds have passed (at least once); its mean rate."""
    import oracle
    lay = oracle.NCHW if layout == "NCHW" else oracle.NHWC
    reps, t, flops = 0, 0.0, 0.0
    while reps == 0 or t < budget_s:
        for p in prepared:
            x, w, b = p.host
            L = p.L
            t0 = time.perf_counter()
            oracle.conv2d(x, w, b, L.stride, L.pad, L.dilation, lay, want_norm=False)
            t += time.perf_counter() - t0
            flops += layer_flops(L, p.Ho, p.Wo, n=x.shape[0])
        reps += 1
    return {"value": flops / t / 1e12, "unit": "TFLOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the first {CPU_SAMPLE_IMAGES} of the 128 images of each of the five layers of the "
                      f"set (full fp64 output of each), {reps} repetition(s), {t:.1f} s"}


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


def sweep(args, flush, rows_out):
    """Every layer shape under every algorithm, then the main-loop ablation;
    rows to stderr and to rows_out."""
    import torch
    import convolution_lowering_amd as cl
    from convolution_lowering_amd.workloads import LAYERS
    rows, ablation = [], []
    steps = max(3, args.steps // 4)
    for name, L in LAYERS.items():
        extra = ("fp16",) if name == "C2" else ()
        extra += ("fp8",) if name in ("C2", "C3c", "C4b", "C4c", "C4d", "C4e") else ()
        for dtype in L.dtypes + extra:
            for layout in ("NCHW", "NHWC"):
                algos = ["auto", "im2col", "direct", "im2win_lds"]
                if name == "C2":
                    algos = ["auto", "indirect", "im2win", "im2col", "direct", "im2win_lds"]
                for algo in algos:
                    try:
                        r = bench_layer(L, dtype, layout, algo, steps, 2, flush)
                    except cl.ConvLowerError as e:
                        if e.code == 2 and (algo == "im2win_lds" or dtype == "fp8"):
                            continue  # shape or layout outside the window-rows-in-LDS loop
                        r = {"layer": name, "dtype": dtype, "layout": layout, "algo": algo, "error": str(e)}
                    rows.append(r)
                    print("# row " + json.dumps(r), file=sys.stderr, flush=True)
    for name, dtype, layout in (("C2", "bf16", "NHWC"), ("C4b", "bf16", "NHWC"), ("C4d", "bf16", "NHWC")):
        L = LAYERS[name]
        for variant in list(cl.MAIN_LOOPS) + list(cl.ABLATIONS):
            cl.force_main_loop(variant)
            try:
                r = bench_layer(L, dtype, layout, "auto", steps, 2, flush)
                a = {"layer": name, "dtype": dtype, "layout": layout, "main_loop": variant, "ms": r["ms"],
                     "tflops": r["tflops"]}
            except cl.ConvLowerError as e:
                a = {"layer": name, "dtype": dtype, "layout": layout, "main_loop": variant, "error": str(e)}
            finally:
                cl.force_main_loop("auto")
            ablation.append(a)
            print("# ablation " + json.dumps(a), file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
    if rows_out:
        with open(rows_out, "w") as fh:
            json.dump({"layers": rows, "ablation": ablation}, fh, indent=1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", choices=["all", "headline"], default="headline",
                    help="all: also the per-layer sweep over every shape and algorithm, and the ablation")
    ap.add_argument("--rows-out", metavar="FILE", help="where --layers all writes its rows (JSON)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clock-warmup", type=float, default=0.5, metavar="SECONDS",
                    help="untimed steps of the set run for this long before the warm-up steps, so the "
                         "shader clock has settled (0: none)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one 256 MiB device copy (scale reference for HBM byte counters)")
    ap.add_argument("--only", metavar="LAYER:LAYOUT[:DTYPE[:ALGO]][,...]",
                    help="time only these layers (algo auto, dtype bf16 unless given), one JSON row each; "
                         "for profiling a few layers' kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path (each GPU would run its own "
              "share of the batch independently)", file=sys.stderr)
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
        for spec in args.only.split(","):
            parts = spec.split(":")
            L = LAYERS[parts[0]]
            row = bench_layer(L, parts[2] if len(parts) > 2 else "bf16", parts[1],
                              parts[3] if len(parts) > 3 else "auto", args.steps, args.warmup, flush)
            print(json.dumps(row), flush=True)
        if args.calibration_copy:
            calibration_copy()
        return

    keep = 0 if args.no_cpu_baseline else CPU_SAMPLE_IMAGES
    prepared = [Prepared(LAYERS[n], HEAD_DTYPE, HEAD_LAYOUT, HEAD_ALGO, keep_host_images=keep) for n in HEAD_SET]
    # The shader clock climbs for tens of milliseconds of matrix work: after
    # memory traffic alone, the 64->128 @112 main loop took 400 us in the
    # first steps and 300 us some thirty steps later.  So the set runs
    # untimed for a while first, until the clock has settled.
    t_end = time.perf_counter() + args.clock_warmup
    while time.perf_counter() < t_end:
        for p in prepared:
            p()
        torch.cuda.synchronize()
    t = time_set(prepared, args.steps, args.warmup, flush)
    total_flops = sum(p.flops for p in prepared)
    per_layer = []
    for p, ms in zip(prepared, t["layer_ms"]):
        r = layer_row(p, ms)
        per_layer.append({"layer": p.L.name, "ms": round(ms, 5), "tflops": round(r["tflops"], 1),
                          "bound": r["roofline"]["bound"], "frac": round(r["roofline"]["frac"], 4),
                          "workspace_bytes": p.ws_bytes, "im2col_bytes": p.im2col})
        print(f"# {p.L.name} {HEAD_DTYPE} {HEAD_LAYOUT} {HEAD_ALGO}: {ms:.4f} ms {r['tflops']:.1f} TFLOPS "
              f"{r['roofline']['bound']} frac {r['roofline']['frac']:.3f}", file=sys.stderr, flush=True)
    value = total_flops / t["ms"] / 1e9
    print(f"# set: {t['ms']:.4f} ms per step, {value:.1f} TFLOPS", file=sys.stderr, flush=True)

    # Roofline entry of the dominant kernel: the main loop (with its fused
    # epilogue) of the dominant layer, timed by its own start/end stamps over
    # a second pass of the same steps (a stamped launch takes a few
    # microseconds longer to dispatch, so the step time comes from the pass
    # without them).
    di = HEAD_SET.index(HEAD_DOMINANT)
    ts = time_set(prepared, args.steps, 0, flush, stamp=di)
    dom = prepared[di]
    rl = roofline(dom.flops, dom.nbytes, ts["kernel_ms"] / 1e3, HEAD_DTYPE)
    rl["traffic"] = measured_traffic(TRAFFIC_KEY)
    rl["kernel"] = f"main loop of {HEAD_DOMINANT} (MFMA implicit GEMM over window rows staged in LDS + fused epilogue)"
    rl["kernel_ms"] = ts["kernel_ms"]
    rl["per_launch_flops"] = dom.flops
    rl["per_launch_algorithmic_bytes"] = dom.nbytes
    print(f"# dominant kernel {HEAD_DOMINANT}: {ts['kernel_ms']:.4f} ms, {rl['achieved']:.1f} {rl['unit']}, "
          f"frac {rl['frac']:.3f}", file=sys.stderr, flush=True)

    if args.calibration_copy:
        calibration_copy()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(prepared, HEAD_LAYOUT)
        print(f"# cpu baseline: {cpu['value']:.4f} TFLOPS on {cpu['cores']} threads", file=sys.stderr, flush=True)
    for p in prepared:
        p.host = None
    del prepared
    torch.cuda.empty_cache()

    if args.layers == "all":
        sweep(args, flush, args.rows_out)

    print(summary_line(value, t["ms"], args.steps, args.warmup, per_layer, rl, cpu))


def summary_line(value, ms_per_step, steps, warmup, per_layer, rl, cpu):
    """The last stdout line: one compact JSON object (a few KB at most)."""
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOPS", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": HEAD_DTYPE,
        "data": "synthetic (seeded torch CPU generator; x ~ U[-1,1], Kaiming-normal w, bias ~ N(0,1)), "
                "MALL flushed before each step (512 MB written, then 512 MB read)",
        "config": {"workload": HEAD_WORKLOAD, "layout": HEAD_LAYOUT, "algo": HEAD_ALGO, "global_batch": 128,
                   "step": "one conv2d_fwd call per layer of the set", "per_layer": per_layer},
        "roofline": rl,
        "cpu_baseline": cpu,
    }
    return json.dumps(line)


if __name__ == "__main__":
    main()
