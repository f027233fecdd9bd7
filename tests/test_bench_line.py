"""The benchmark's last stdout line stays one compact JSON object with the
fields its readers parse (no GPU needed: the line is built from stand-in
figures)."""
import json

import bench


def test_summary_line_is_compact_and_complete():
    per_layer = [{"layer": n, "ms": 0.123456, "tflops": 1234.5, "bound": "mfma", "frac": 0.4938,
                  "workspace_bytes": 123456789, "im2col_bytes": 1849688064} for n in bench.HEAD_SET]
    rl = bench.roofline(2.3676e11, 6.167e8, 2.5e-4, "bf16")
    rl.update({"traffic": 6.2e8, "kernel": "main loop of C4b (MFMA implicit GEMM over window rows staged in LDS "
               "+ fused epilogue)", "kernel_ms": 0.25, "per_launch_flops": 2.3676e11,
               "per_launch_algorithmic_bytes": 6.167e8})
    cpu = {"value": 0.0331, "unit": "TFLOPS", "cores": 16, "kind": "oracle",
           "sample": "the first 16 of the 128 images of each of the five layers of the set (full fp64 output "
                     "of each), 3 repetition(s), 12.3 s"}
    line = bench.summary_line(987.6, 1.234, 20, 5, per_layer, rl, cpu)
    assert "\n" not in line and len(line) < 4096, len(line)
    rec = json.loads(line)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in rec, k
    assert rec["config"]["workload"].startswith("VGG-16")
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rec["roofline"], k
    assert rec["roofline"]["bound"] == "mfma" and abs(rec["roofline"]["frac"] - 2.3676e11 / 2.5e-4 / 2.5e15) < 1e-9
    assert rec["cpu_baseline"]["kind"] == "oracle"
