"""conv2d_fwd_noalloc against conv2d_fwd, through the C ABI.

The no-allocation entry point runs the same plan and kernels as conv2d_fwd
with the library's per-GPU scratch array as the workspace, so its output must
equal conv2d_fwd's bit for bit.  Each case makes two calls in a row on the
same scratch array, the second with a smaller batch, so the second call
starts from whatever the first left there.
"""
import sys
from dataclasses import replace

import pytest
import torch

import convolution_lowering_amd as cl
from convolution_lowering_amd.workloads import LAYERS, make_inputs

pytestmark = pytest.mark.gpu

# (layer, dtype, layout, algo, first N, second N): the lowering copy plus the
# window-row loop; split-K partials (the dense layer); the indirection
# buffer; the padded window tensor; the NCHW 1x1 halves.
CASES = [
    ("C2", "bf16", "NCHW", "auto", 32, 3),
    ("C5c", "fp32", "NHWC", "auto", 16, 5),
    ("C3e", "bf16", "NHWC", "indirect", 16, 2),
    ("C5a", "bf16", "NCHW", "auto", 16, 3),
    ("C3b", "bf16", "NCHW", "auto", 16, 3),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}" for c in CASES])
def test_noalloc_matches_fwd_twice(case):
    name, dtype, layout, algo, n1, n2 = case
    L = LAYERS[name]
    for n in (n1, n2):
        need = cl.workspace_size(n, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation, layout, dtype,
                                 algo)
        assert need <= cl.NOALLOC_SCRATCH_BYTES, (name, n, need)
        _say(f"[gpu] noalloc {name} {dtype} {layout} {algo} N={n} workspace={need}")
        x, w, b = make_inputs(L, dtype, layout, N=n)
        x, w, b = x.cuda(), w.cuda(), b.cuda()
        ref = cl.conv2d_fwd(x, w, b, L.stride, L.pad, L.dilation, layout, algo)
        out = torch.full_like(ref, float("nan"))
        cl.conv2d_fwd_noalloc(x, w, b, out, L.stride, L.pad, L.dilation, layout, algo)
        torch.cuda.synchronize()
        bits = torch.int32 if out.dtype == torch.float32 else torch.int16
        assert torch.equal(out.view(bits), ref.view(bits)), f"{name} N={n}: no-allocation output differs from conv2d_fwd"


def test_noalloc_on_a_side_stream():
    """The work goes to the caller's stream (default priority)."""
    L = LAYERS["C2"]
    x, w, b = make_inputs(L, "bf16", "NCHW", N=4)
    x, w, b = x.cuda(), w.cuda(), b.cuda()
    ref = cl.conv2d_fwd(x, w, b, L.stride, L.pad, L.dilation, "NCHW", "auto")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    out = torch.zeros_like(ref)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cl.conv2d_fwd_noalloc(x, w, b, out, L.stride, L.pad, L.dilation, "NCHW", "auto", stream=s)
    s.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_noalloc_without_the_stream_k_regions():
    """Where the stream-K partial tiles would take the workspace past the
    scratch array, the no-allocation call runs the one-tile-per-block loop
    instead: fp32 3x3 256->128 @28, NCHW, N = 88 (135 tiles of 512 x 128),
    138.9 MB of workspace with the partial tiles and 71.8 MB without.  On
    small-integer inputs every partial sum is exact, so the two calls give
    the same bits although they add in different orders."""
    L = replace(LAYERS["C4d"], Co=128, N=88)
    need = cl.workspace_size(L.N, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation, "NCHW", "fp32",
                             "auto")
    assert need > cl.NOALLOC_SCRATCH_BYTES >= need - 256 * 512 * 128 * 4 - 1024
    _say(f"[gpu] noalloc without stream-K: fp32 256->128@28 N=88 workspace={need}")
    x, w, b = make_inputs(L, "fp32", "NCHW", integer=True)
    x, w, b = x.cuda(), w.cuda(), b.cuda()
    ref = cl.conv2d_fwd(x, w, b, L.stride, L.pad, L.dilation, "NCHW", "auto")
    out = torch.full_like(ref, float("nan"))
    cl.conv2d_fwd_noalloc(x, w, b, out, L.stride, L.pad, L.dilation, "NCHW", "auto")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
