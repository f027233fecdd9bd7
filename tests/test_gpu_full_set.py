"""Whole-output parity at full size for the layer set the benchmark times.

Every output of every layer of the VGG-16-shaped 3x3 set (N=128, the
benchmark's shapes and launch configuration) is compared with the fp64
oracle, in both layouts:
- bf16 on the benchmark's own inputs, to max |y - y_ref| / D <= 8e-3;
- fp32 on small-integer inputs ({-3..3}: every product and partial sum is
  an exact float32 integer), bit for bit.
The comparison runs image by image so the host holds one fp64 copy of y.
"""
import sys

import numpy as np
import pytest
import torch

import convolution_lowering_amd as cl
import oracle
from convolution_lowering_amd.workloads import LAYERS, make_inputs

pytestmark = pytest.mark.gpu

SET = ("C4a", "C4b", "C4c", "C4d", "C4e")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu(L, x, w, b, layout):
    y = cl.conv2d_fwd(x.cuda(), w.cuda(), b.cuda(), L.stride, L.pad, L.dilation, layout, "auto")
    torch.cuda.synchronize()
    y = y.cpu()
    return y if layout == "NCHW" else y.permute(0, 3, 1, 2)


@pytest.mark.parametrize("name", SET)
def test_full_layer_bf16_whole_output(name):
    L = LAYERS[name]
    x, w, b = make_inputs(L, "bf16", "NCHW")
    _say(f"[gpu] full {name} bf16 N={L.N}: oracle")
    y_ref, dn = oracle.conv2d(x, w, b, L.stride, L.pad, L.dilation, oracle.NCHW)
    for layout in ("NCHW", "NHWC"):
        _say(f"[gpu] full {name} bf16 {layout}")
        if layout == "NHWC":
            xl, wl = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
        else:
            xl, wl = x, w
        y = _gpu(L, xl, wl, b, layout)
        worst = 0.0
        for n in range(L.N):
            yn = y[n].double().numpy()
            assert np.all(np.isfinite(yn)), (name, layout, n)
            worst = max(worst, float(np.max(np.abs(yn - y_ref[n]) / dn[n])))
        assert worst <= 8e-3, f"{name} {layout}: normalised error {worst:.3e}"
        _say(f"[gpu] full {name} bf16 {layout}: worst normalised error {worst:.3e}")
        del y


@pytest.mark.parametrize("name", SET)
def test_full_layer_fp32_integer_bitwise(name):
    L = LAYERS[name]
    x, w, b = make_inputs(L, "fp32", "NCHW", integer=True)
    _say(f"[gpu] full {name} fp32 integer N={L.N}: oracle")
    y_ref = oracle.conv2d(x, w, b, L.stride, L.pad, L.dilation, oracle.NCHW, want_norm=False)
    for layout in ("NCHW", "NHWC"):
        _say(f"[gpu] full {name} fp32 integer {layout}")
        if layout == "NHWC":
            xl, wl = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
        else:
            xl, wl = x, w
        y = _gpu(L, xl, wl, b, layout)
        for n in range(L.N):
            yn = y[n].double().numpy()
            bad = int(np.count_nonzero(yn != y_ref[n]))
            assert bad == 0, f"{name} {layout} image {n}: {bad} outputs differ from the exact result"
        del y
