"""The stream-K form of the one-block-per-CU window-row loop, against the oracle.

The calls ask for the window rows in LDS (IM2WIN_LDS): below 256 tiles of
256 x 128 AUTO takes another lowering.

A 3x3 512->512 layer at 14x14 with N = 64 has 100 output tiles of 512 x 128
for 256 blocks: every tile's K steps are split over about three blocks, so
tiles are finished from the partial sums of one or two other blocks.  With
N = 40 every call takes the same form except bf16 NCHW, whose channels-last
copy leaves no room below the im2col footprint: it keeps one tile per block.
Whole outputs are compared with the fp64 oracle: bf16 to the normalised
bound, fp32 on small-integer inputs bit for bit (every partial sum is an
exact integer, so the order the blocks add them in cannot matter).
"""
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import convolution_lowering_amd as cl
import oracle
from convolution_lowering_amd.workloads import LAYERS, make_inputs

pytestmark = pytest.mark.gpu

SK_BYTES = 256 * 512 * 128 * 4  # the partial tiles alone


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _layer(n):
    return LAYERS["C4e"].with_batch(n)


def _call(L, x, w, b, layout):
    if layout == "NHWC":
        x, w = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
    y = cl.conv2d_fwd(x.cuda(), w.cuda(), b.cuda(), L.stride, L.pad, L.dilation, layout, "im2win_lds")
    torch.cuda.synchronize()
    y = y.cpu()
    return y if layout == "NCHW" else y.permute(0, 3, 1, 2)


@pytest.mark.parametrize("n,layout", [(64, "NHWC"), (64, "NCHW"), (40, "NHWC"), (40, "NCHW")])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_stream_k_whole_output(n, layout, dtype):
    L = _layer(n)
    # bf16 NCHW at N = 40: copy, weights and partial tiles would pass im2col.
    stream_k = not (n == 40 and layout == "NCHW" and dtype == "bf16")
    ws = cl.workspace_size(L.N, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation, layout, dtype,
                           "im2win_lds")
    assert (ws >= SK_BYTES) == stream_k, ws
    integer = dtype == "fp32"
    x, w, b = make_inputs(L, dtype, "NCHW", integer=integer)
    _say(f"[gpu] stream-K {L.C}->{L.Co}@{L.H} N={n} {layout} {dtype} workspace={ws}")
    y = _call(L, x, w, b, layout)
    worst = 0.0
    for n0 in range(0, n, 16):
        sl = slice(n0, min(n0 + 16, n))
        if integer:
            y_ref = oracle.conv2d(x[sl], w, b, L.stride, L.pad, L.dilation, oracle.NCHW, want_norm=False)
            bad = int(np.count_nonzero(y[sl].double().numpy() != y_ref))
            assert bad == 0, f"images {n0}..: {bad} outputs differ from the exact result"
        else:
            y_ref, dn = oracle.conv2d(x[sl], w, b, L.stride, L.pad, L.dilation, oracle.NCHW)
            yn = y[sl].double().numpy()
            assert np.all(np.isfinite(yn))
            worst = max(worst, float(np.max(np.abs(yn - y_ref) / dn)))
    assert worst <= 8e-3, f"normalised error {worst:.3e}"
    _say(f"[gpu]   worst normalised error {worst:.3e}")


@pytest.mark.parametrize("layout,dtype", [("NHWC", "bf16"), ("NHWC", "fp32"), ("NCHW", "fp32")])
def test_stream_k_ragged_tiles(layout, dtype):
    """3x3 256->200 @14, N = 128: the last of 49 pixel tiles is partial and
    the second of two channel tiles holds 72 of its 128 channels (98 tiles
    split over 256 blocks)."""
    L = replace(_layer(128), C=256, Co=200)
    ws = cl.workspace_size(L.N, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation, layout, dtype,
                           "im2win_lds")
    assert ws >= SK_BYTES, ws
    integer = dtype == "fp32"
    x, w, b = make_inputs(L, dtype, "NCHW", integer=integer)
    _say(f"[gpu] stream-K ragged {L.C}->{L.Co}@{L.H} N={L.N} {layout} {dtype} workspace={ws}")
    y = _call(L, x, w, b, layout)
    worst = 0.0
    for n0 in range(0, L.N, 32):
        sl = slice(n0, min(n0 + 32, L.N))
        if integer:
            y_ref = oracle.conv2d(x[sl], w, b, L.stride, L.pad, L.dilation, oracle.NCHW, want_norm=False)
            bad = int(np.count_nonzero(y[sl].double().numpy() != y_ref))
            assert bad == 0, f"images {n0}..: {bad} outputs differ from the exact result"
        else:
            y_ref, dn = oracle.conv2d(x[sl], w, b, L.stride, L.pad, L.dilation, oracle.NCHW)
            yn = y[sl].double().numpy()
            assert np.all(np.isfinite(yn))
            worst = max(worst, float(np.max(np.abs(yn - y_ref) / dn)))
    assert worst <= 8e-3, f"normalised error {worst:.3e}"
    _say(f"[gpu]   worst normalised error {worst:.3e}")


def test_stream_k_fp16():
    """fp16 runs its own instantiation of the loop: N = 64, channels-last,
    against the oracle to the fp16 bound (1e-3 normalised)."""
    L = _layer(64)
    ws = cl.workspace_size(L.N, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation, "NHWC", "fp16",
                           "im2win_lds")
    assert ws >= SK_BYTES, ws
    x, w, b = make_inputs(L, "fp16", "NCHW")
    _say(f"[gpu] stream-K fp16 N=64 NHWC workspace={ws}")
    y = _call(L, x, w, b, "NHWC")
    worst = 0.0
    for n0 in range(0, L.N, 16):
        sl = slice(n0, n0 + 16)
        y_ref, dn = oracle.conv2d(x[sl], w, b, L.stride, L.pad, L.dilation, oracle.NCHW)
        yn = y[sl].double().numpy()
        assert np.all(np.isfinite(yn))
        worst = max(worst, float(np.max(np.abs(yn - y_ref) / dn)))
    assert worst <= 1e-3, f"normalised error {worst:.3e}"
    _say(f"[gpu]   worst normalised error {worst:.3e}")


def test_stream_k_without_bias():
    """No bias: the epilogues of whole, finished and split tiles add nothing
    (N = 64, channels-last, fp32 on small-integer inputs: exact)."""
    L = _layer(64)
    x, w, _ = make_inputs(L, "fp32", "NCHW", integer=True)
    _say("[gpu] stream-K without bias N=64 NHWC fp32")
    xl, wl = x.permute(0, 2, 3, 1).contiguous().cuda(), w.permute(0, 2, 3, 1).contiguous().cuda()
    y = cl.conv2d_fwd(xl, wl, None, L.stride, L.pad, L.dilation, "NHWC", "im2win_lds")
    torch.cuda.synchronize()
    y = y.cpu().permute(0, 3, 1, 2)
    for n0 in range(0, L.N, 16):
        sl = slice(n0, n0 + 16)
        y_ref = oracle.conv2d(x[sl], w, None, L.stride, L.pad, L.dilation, oracle.NCHW, want_norm=False)
        bad = int(np.count_nonzero(y[sl].double().numpy() != y_ref))
        assert bad == 0, f"images {n0}..: {bad} outputs differ from the exact result"


def test_stream_k_runs_are_bitwise_equal():
    """The finishing blocks add the others' sums in a fixed order: two calls
    give the same bits."""
    L = _layer(64)
    x, w, b = make_inputs(L, "bf16", "NHWC")
    _say("[gpu] stream-K determinism N=64 NHWC bf16")
    x, w, b = x.cuda(), w.cuda(), b.cuda()
    y1 = cl.conv2d_fwd(x, w, b, L.stride, L.pad, L.dilation, "NHWC", "im2win_lds")
    y2 = cl.conv2d_fwd(x, w, b, L.stride, L.pad, L.dilation, "NHWC", "im2win_lds")
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
