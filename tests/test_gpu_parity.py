"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Criterion: err = max |y_gpu - y_ref| / D with D = sum |x||w| + |bias| over
each output's terms; err <= 1e-5 for fp32 and <= 8e-3 for bf16 (inputs are
the bf16-rounded values, so only the kernel's own rounding is charged).
Where D = 0 (a window wholly in the padding, no bias) y must be exactly 0.
With small-integer inputs every product and partial sum is exact in fp32,
so there the fp32 output must equal the exact result bit for bit and the
bf16 output must equal the exact result rounded once to nearest-even.
"""
import sys

import numpy as np
import pytest
import torch

import convolution_lowering_amd as cl
import oracle
from convolution_lowering_amd.workloads import LAYERS, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 8e-3, "fp16": 1e-3}
DEV = "cuda"
_ORACLE_CACHE = {}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle_full(L, dtype, n, bias=True, integer=False):
    key = (L.name, dtype, n, bias, integer)
    if key not in _ORACLE_CACHE:
        x, w, b = make_inputs(L, dtype, "NCHW", N=n, bias=bias, integer=integer)
        y, dn = oracle.conv2d(x, w, b, L.stride, L.pad, L.dilation, oracle.NCHW)
        _ORACLE_CACHE[key] = (y, dn)
    return _ORACLE_CACHE[key]


def _to_nchw(t, layout):
    return t if layout == "NCHW" else t.permute(0, 3, 1, 2)


def _run(L, dtype, layout, algo, n, bias=True, integer=False):
    x, w, b = make_inputs(L, dtype, layout, N=n, bias=bias, integer=integer)
    _say(f"[gpu] {L.name} {dtype} {layout} {algo} N={n} bias={bias} integer={integer}")
    xd, wd = x.to(DEV), w.to(DEV)
    bd = b.to(DEV) if b is not None else None
    y = cl.conv2d_fwd(xd, wd, bd, L.stride, L.pad, L.dilation, layout, algo)
    torch.cuda.synchronize()
    return y


def _assert_parity(y_gpu, y_ref, dn, dtype, what):
    y = y_gpu.double().cpu().numpy()
    assert y.shape == y_ref.shape, what
    assert np.all(np.isfinite(y)), what
    zero = dn == 0
    assert np.all(y[zero] == 0), what
    err = np.abs(y - y_ref)[~zero] / dn[~zero]
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dtype], f"{what}: normalised error {worst:.3e} > {TOL[dtype]:.0e}"
    return worst


# --- whole-output parity at reduced batch (several tiles and a ragged tail) ----

SMALL_N = {"C1": 2, "C2": 2, "C3a": 1, "C3b": 2, "C3c": 2, "C3d": 2, "C3e": 2, "C4a": 1, "C4b": 1,
           "C4c": 1, "C4d": 1, "C4e": 2, "C5a": 2, "C5b": 2, "C5c": 16}


def _rowwin_eligible(L, dtype):
    """The shapes CONV_ALGO_IM2WIN_LDS serves (the header's rule)."""
    Wo = oracle.out_size(L.W, L.KW, L.stride, L.pad, L.dilation)
    return (L.stride == 1 and L.dilation == 1 and L.KW == 3 and L.C % (16 if dtype == "fp32" else 32) == 0
            and 255 // Wo + 2 <= 32)


def _cases():
    out = []
    for name, L in LAYERS.items():
        plain = (L.KH == L.KW == 1 and L.stride == 1 and L.pad == 0) or (L.KH == L.H and L.KW == L.W and L.pad == 0)
        algos = ["auto", "indirect", "im2win", "im2col", "direct"] + (["gemm"] if plain else [])
        for dtype in sorted(set(L.dtypes) | {"fp32", "bf16", "fp16"} if name in ("C1", "C2", "C5a", "C5b", "C5c")
                            else L.dtypes):
            for layout in ("NCHW", "NHWC"):
                for algo in algos + (["im2win_lds"] if _rowwin_eligible(L, dtype) else []):
                    out.append((name, dtype, layout, algo))
    return out


@pytest.mark.parametrize("name,dtype,layout,algo", _cases())
def test_parity_reduced_batch(name, dtype, layout, algo):
    L = LAYERS[name]
    n = SMALL_N[name]
    y = _run(L, dtype, layout, algo, n)
    y_ref, dn = _oracle_full(L, dtype, n)
    _assert_parity(_to_nchw(y, layout), y_ref, dn, dtype, f"{name} {dtype} {layout} {algo}")


@pytest.mark.parametrize("name", ["C1", "C2", "C5a", "C5c"])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("algo", ["auto", "im2win"])
def test_parity_without_bias(name, layout, algo):
    L = LAYERS[name]
    n = SMALL_N[name]
    y = _run(L, "fp32", layout, algo, n, bias=False)
    y_ref, dn = _oracle_full(L, "fp32", n, bias=False)
    _assert_parity(_to_nchw(y, layout), y_ref, dn, "fp32", f"{name} no-bias {layout} {algo}")


@pytest.mark.parametrize("name", ["C1", "C2", "C3a", "C3e", "C4a", "C5a", "C5b", "C5c"])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("algo", ["auto", "indirect", "im2win"])
def test_integer_inputs_exact(name, layout, algo):
    L = LAYERS[name]
    n = SMALL_N[name]
    y_ref, _ = _oracle_full(L, "fp32", n, integer=True)
    y32 = _to_nchw(_run(L, "fp32", layout, algo, n, integer=True), layout).double().cpu().numpy()
    assert np.array_equal(y32, y_ref), f"{name} {layout} {algo}: fp32 not exact"
    yb = _to_nchw(_run(L, "bf16", layout, algo, n, integer=True), layout).float().cpu()
    exp = torch.from_numpy(y_ref).float().to(torch.bfloat16).float()
    assert torch.equal(yb, exp), f"{name} {layout} {algo}: bf16 not the rounded exact result"
    # fp16: the exact result (an integer well inside fp16's range) rounded
    # once to nearest, ties to even
    yh = _to_nchw(_run(L, "fp16", layout, algo, n, integer=True), layout).float().cpu()
    exp = torch.from_numpy(y_ref).float().to(torch.float16).float()
    assert torch.equal(yh, exp), f"{name} {layout} {algo}: fp16 not the rounded exact result"


# --- full-size layers, in the configuration the benchmark times -------------

def _sample_points(L, n, count, seed):
    Ho = oracle.out_size(L.H, L.KH, L.stride, L.pad, L.dilation)
    Wo = oracle.out_size(L.W, L.KW, L.stride, L.pad, L.dilation)
    rng = np.random.default_rng(seed)
    pts = np.stack([rng.integers(0, n, count), rng.integers(0, L.Co, count),
                    rng.integers(0, Ho, count), rng.integers(0, Wo, count)], 1)
    corners = [(a, b, c, d) for a in (0, n - 1) for b in (0, L.Co - 1) for c in (0, Ho - 1) for d in (0, Wo - 1)]
    return np.concatenate([pts, np.array(corners)]).astype(np.int32)


def _full_cases():
    out = []
    for name, L in LAYERS.items():
        for dtype in L.dtypes:
            for layout in ("NCHW", "NHWC"):
                out.append((name, dtype, layout, "auto"))
    for algo in ("indirect", "im2win"):
        for layout in ("NCHW", "NHWC"):
            out.append(("C2", "bf16", layout, algo))
    for layout in ("NCHW", "NHWC"):  # the window-row loop's 256 x 64 tile (64 output channels)
        out.append(("C3c", "bf16", layout, "im2win_lds"))
    return out


@pytest.mark.parametrize("name,dtype,layout,algo", _full_cases())
def test_parity_full_size_sampled(name, dtype, layout, algo):
    L = LAYERS[name]
    x, w, b = make_inputs(L, dtype, layout)
    _say(f"[gpu] full {name} {dtype} {layout} {algo} N={L.N}")
    y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), L.stride, L.pad, L.dilation, layout, algo)
    torch.cuda.synchronize()
    pts = _sample_points(L, L.N, 3000, L.seed)
    yn = _to_nchw(y, layout)
    idx = torch.from_numpy(pts.astype(np.int64)).to(DEV)
    got = yn[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].double().cpu().numpy()
    lay = oracle.NCHW if layout == "NCHW" else oracle.NHWC
    ref, dn = oracle.conv2d_points(x, w, b, pts, L.stride, L.pad, L.dilation, lay)
    assert np.all(np.isfinite(y.float().abs().amax().cpu().numpy()))
    err = np.abs(got - ref) / np.where(dn > 0, dn, 1.0)
    assert float(err.max()) <= TOL[dtype], f"{name}: {err.max():.3e}"


@pytest.mark.parametrize("name", ["C2", "C3a", "C4a", "C4c", "C4d", "C4e", "C5a", "C5c"])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_full_size_integer_exact_sampled(name, layout):
    """Bit-exact at full size: integer inputs make the exact result the only
    correct fp32 answer at every sampled output."""
    L = LAYERS[name]
    x, w, b = make_inputs(L, "fp32", layout, integer=True)
    _say(f"[gpu] full-int {name} {layout}")
    y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), L.stride, L.pad, L.dilation, layout, "auto")
    torch.cuda.synchronize()
    pts = _sample_points(L, L.N, 2000, L.seed + 1)
    yn = _to_nchw(y, layout)
    idx = torch.from_numpy(pts.astype(np.int64)).to(DEV)
    got = yn[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].double().cpu().numpy()
    lay = oracle.NCHW if layout == "NCHW" else oracle.NHWC
    ref, _ = oracle.conv2d_points(x, w, b, pts, L.stride, L.pad, L.dilation, lay)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_many_tiles_odd_planes_sampled(layout, dtype):
    """More than 512 output tiles select the 512-thread main loop; planes of
    225 pixels (odd) make its NCHW stores go element by element.  fp32 runs
    on integer inputs and must be exact; bf16 within the tolerance."""
    from convolution_lowering_amd.workloads import Layer
    L = Layer("many-tiles-odd-planes", 160, 64, 15, 15, 512, 3, 3, 1, 1, 1, seed=91)
    integer = dtype == "fp32"
    x, w, b = make_inputs(L, dtype, layout, integer=integer)
    _say(f"[gpu] many-tiles {dtype} {layout}")
    y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), L.stride, L.pad, L.dilation, layout, "indirect")
    torch.cuda.synchronize()
    pts = _sample_points(L, L.N, 3000, L.seed)
    yn = _to_nchw(y, layout)
    idx = torch.from_numpy(pts.astype(np.int64)).to(DEV)
    got = yn[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].double().cpu().numpy()
    lay = oracle.NCHW if layout == "NCHW" else oracle.NHWC
    ref, dn = oracle.conv2d_points(x, w, b, pts, L.stride, L.pad, L.dilation, lay)
    if integer:
        assert np.array_equal(got, ref)
    else:
        err = np.abs(got - ref) / np.where(dn > 0, dn, 1.0)
        assert float(err.max()) <= TOL[dtype], f"{err.max():.3e}"


@pytest.mark.parametrize("shape", [(8, 256, 28), (16, 32, 56), (24, 32, 56)])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_window_rows_both_block_forms(shape, layout, dtype):
    """256 output channels, 3x3: N=8, C=256 at 28x28 (26 tiles of 512 x 128,
    72 taps) takes the one-block ping-pong form; C=32 at 56x56 (9 taps), at
    N=16 (one round of 512-row tiles) and N=24 (more), takes two 256 x 128
    blocks per compute unit.  The whole output is compared: fp32 on integer
    inputs bit for bit, bf16 within the tolerance."""
    from convolution_lowering_amd.workloads import Layer
    n, c, hw = shape
    L = Layer(f"rowwin-forms-{n}-{c}", n, c, hw, hw, 256, 3, 3, 1, 1, 1, seed=97)
    integer = dtype == "fp32"
    x, w, b = make_inputs(L, dtype, layout, integer=integer)
    _say(f"[gpu] rowwin-forms N={n} C={c} {dtype} {layout}")
    y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), L.stride, L.pad, L.dilation, layout, "im2win_lds")
    torch.cuda.synchronize()
    xr, wr, br = make_inputs(L, dtype, "NCHW", integer=integer)
    y_ref, dn = oracle.conv2d(xr, wr, br, L.stride, L.pad, L.dilation, oracle.NCHW)
    yn = _to_nchw(y, layout)
    if integer:
        assert np.array_equal(yn.double().cpu().numpy(), y_ref)
    else:
        _assert_parity(yn, y_ref, dn, dtype, f"rowwin forms N={n} C={c}")


ROWWIN64_CASES = [
    # name, N, C, H, W, Co
    ("co64-ragged", 2, 64, 30, 29, 64),     # 1740 pixels: 7 tiles of 256, the last ragged
    ("co48", 3, 32, 17, 60, 48),            # 48 of the tile's 64 channels
    ("co1-wide", 1, 96, 9, 130, 1),         # one output channel, 130-wide rows
    ("co64-many", 2, 32, 56, 56, 64),       # 25 tiles
]


@pytest.mark.parametrize("case", ROWWIN64_CASES, ids=[c[0] for c in ROWWIN64_CASES])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_window_rows_64_wide_tile(case, layout, dtype):
    """3x3 stride-1 layers with at most 64 output channels take the window-row
    loop's 256 x 64 block tile under "im2win_lds" (four 64 x 64 wavefront
    tiles stacked along M).  The whole output is compared: fp32 on integer
    inputs bit for bit, bf16 within the tolerance."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co = case
    L = Layer(f"rowwin64-{name}", N, C, H, W, Co, 3, 3, 1, 1, 1, seed=101)
    assert _rowwin_eligible(L, dtype)
    integer = dtype == "fp32"
    x, w, b = make_inputs(L, dtype, layout, integer=integer)
    _say(f"[gpu] rowwin64 {name} {dtype} {layout}")
    y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), 1, 1, 1, layout, "im2win_lds")
    torch.cuda.synchronize()
    xr, wr, br = make_inputs(L, dtype, "NCHW", integer=integer)
    y_ref, dn = oracle.conv2d(xr, wr, br, 1, 1, 1, oracle.NCHW)
    yn = _to_nchw(y, layout)
    if integer:
        assert np.array_equal(yn.double().cpu().numpy(), y_ref)
    else:
        _assert_parity(yn, y_ref, dn, dtype, f"rowwin64 {name}")


PATCH_CASES = [
    # name, N, C, H, W, Co, KH, KW, s, p, d
    ("c1-3x3", 2, 1, 17, 19, 40, 3, 3, 1, 1, 1),
    ("c2-5x5-s2-d2", 2, 2, 23, 21, 70, 5, 5, 2, 3, 2),     # two channel tiles, the second ragged
    ("c3-7x7-s2", 2, 3, 30, 33, 64, 7, 7, 2, 3, 1),        # the stem's shape, small
    ("c4-1x2", 3, 4, 9, 40, 5, 1, 2, 1, 0, 1),             # 5 output channels, 39-wide rows
    ("c3-wide-rows", 1, 3, 6, 130, 33, 3, 3, 1, 1, 1),     # 130-wide rows: a ragged last fragment
    ("c3-odd-planes", 2, 3, 15, 15, 64, 3, 3, 1, 1, 1),    # 225-pixel planes: element stores
]


@pytest.mark.parametrize("case", PATCH_CASES, ids=[c[0] for c in PATCH_CASES])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_patch_small_channels(case, dtype, layout):
    """PATCH (inputs with at most four channels, patches staged in LDS)
    against the whole oracle output: fp32 on integer inputs bit for bit, the
    16-bit types within the tolerance.  Shapes outside it (fp32 with more
    than 32 taps) are refused with CONV_ERR_UNSUPPORTED."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co, KH, KW, s, p, d = case
    L = Layer(name, N, C, H, W, Co, KH, KW, s, p, d, seed=83)
    if dtype == "fp32" and KH * KW > 32:
        with pytest.raises(cl.ConvLowerError):
            cl.workspace_size(N, C, H, W, Co, KH, KW, s, p, d, layout, dtype, "patch")
        return
    integer = dtype == "fp32"
    x, w, b = make_inputs(L, dtype, layout, integer=integer)
    _say(f"[gpu] patch {name} {dtype} {layout}")
    assert cl.workspace_size(N, C, H, W, Co, KH, KW, s, p, d, layout, dtype, "patch") == 0
    y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), s, p, d, layout, "patch")
    torch.cuda.synchronize()
    xr, wr, br = make_inputs(L, dtype, "NCHW", integer=integer)
    y_ref, dn = oracle.conv2d(xr, wr, br, s, p, d, oracle.NCHW)
    yn = _to_nchw(y, layout)
    if integer:
        assert np.array_equal(yn.double().cpu().numpy(), y_ref)
    else:
        _assert_parity(yn, y_ref, dn, dtype, f"patch {name}")


# Rows of a multiple of 8 columns, 16-bit types: PATCH stages the input in
# 16-byte loads of 8 columns.  Paddings past a load's width, a staged width
# short of the last input column (stride 2), several images per grid pass.
PATCH_VEC_CASES = [
    # name, N, C, H, W, Co, KH, KW, s, p, d
    ("c1-3x3-w16", 3, 1, 11, 16, 40, 3, 3, 1, 1, 1),
    ("c2-5x5-s2-d2-w24", 2, 2, 19, 24, 70, 5, 5, 2, 3, 2),
    ("c3-7x7-s2-w32", 2, 3, 30, 32, 64, 7, 7, 2, 3, 1),
    ("c3-3x3-w128", 2, 3, 9, 128, 33, 3, 3, 1, 1, 1),
    ("c3-3x3-s2-p0-w24", 4, 3, 13, 24, 64, 3, 3, 2, 0, 1),   # staged width 23: column 23 unused
    ("c4-3x3-p9-w8", 2, 4, 7, 8, 20, 3, 3, 1, 9, 1),          # padding wider than a load
    ("c2-1x1-w48", 5, 2, 5, 48, 64, 1, 1, 1, 0, 1),
]


@pytest.mark.parametrize("case", PATCH_VEC_CASES, ids=[c[0] for c in PATCH_VEC_CASES])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_patch_vector_staging(case, dtype, layout):
    """The 16-byte staging against the whole oracle output (integer inputs:
    the exact result rounded once) and against the element-by-element
    staging, which an x one element off 16-byte alignment selects: the same
    bits."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co, KH, KW, s, p, d = case
    L = Layer(name, N, C, H, W, Co, KH, KW, s, p, d, seed=91)
    for integer in (True, False):
        x, w, b = make_inputs(L, dtype, layout, integer=integer)
        _say(f"[gpu] patch 16-byte staging {name} {dtype} {layout} integer={integer}")
        y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), s, p, d, layout, "patch")
        y2 = cl.conv2d_fwd(_misaligned_copy(x), w.to(DEV), b.to(DEV), s, p, d, layout, "patch")
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), name
        xr, wr, br = make_inputs(L, dtype, "NCHW", integer=integer)
        y_ref, dn = oracle.conv2d(xr, wr, br, s, p, d, oracle.NCHW)
        yn = _to_nchw(y, layout)
        if integer:
            exact = torch.from_numpy(y_ref).float().to(y.dtype).float()
            assert torch.equal(yn.float().cpu(), exact), name
        else:
            _assert_parity(yn, y_ref, dn, dtype, f"patch 16-byte staging {name}")


POINTWISE_CASES = [
    # name, N, C, H, W, Co
    ("c64-co72", 3, 64, 7, 9, 72),        # 189 pixel rows (ragged last unit), a second 8-channel chunk
    ("c128-co40", 2, 128, 5, 13, 40),     # 130 rows, one partial chunk
    ("c256-co64", 2, 256, 11, 12, 64),    # 264 rows
    ("c256-co128", 1, 256, 3, 5, 128),    # 15 rows: less than one unit
    ("c64-co512", 2, 64, 6, 6, 512),      # the most weights the kernel holds (64 KB)
    ("c256-co120", 4, 256, 9, 7, 120),    # 120 = 64 + 56 channels
]


@pytest.mark.parametrize("case", POINTWISE_CASES, ids=[c[0] for c in POINTWISE_CASES])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("shift", [0, 1])
def test_pointwise_1x1_channels_last(case, dtype, bias, shift):
    """1x1, unit-stride, unpadded channels-last layers in 16-bit types (the
    input itself is the GEMM operand) with ragged pixel counts and channel
    counts off the 64-channel tile, aligned (shift=0) and with x and y one
    element off 16-byte alignment (shift=1): "auto" and "gemm" against the
    whole oracle output, and the two calls write the same bits."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co = case
    L = Layer(name, N, C, H, W, Co, 1, 1, 1, 0, 1, seed=87)
    x, w, b = make_inputs(L, dtype, "NHWC", bias=bias)
    _say(f"[gpu] pointwise {name} {dtype} bias={bias} shift={shift}")
    assert cl.workspace_size(N, C, H, W, Co, 1, 1, 1, 0, 1, "NHWC", dtype, "gemm") == 0
    if shift:
        xd = _misaligned_copy(x)
        y = _misaligned_copy(torch.zeros((N, H, W, Co), dtype=x.dtype))
    else:
        xd = x.to(DEV)
        y = torch.zeros((N, H, W, Co), dtype=x.dtype, device=DEV)
    bd = b.to(DEV) if b is not None else None
    cl.conv2d_fwd(xd, w.to(DEV), bd, 1, 0, 1, "NHWC", "auto", out=y)
    y2 = torch.full_like(y, 7.0)
    cl.conv2d_fwd(xd, w.to(DEV), bd, 1, 0, 1, "NHWC", "gemm", out=y2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    xr, wr, br = make_inputs(L, dtype, "NCHW", bias=bias)
    y_ref, dn = oracle.conv2d(xr, wr, br, 1, 0, 1, oracle.NCHW)
    _assert_parity(_to_nchw(y, "NHWC"), y_ref, dn, dtype, f"pointwise {name} {dtype}")


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_patch_misaligned_and_twice(layout, dtype):
    """PATCH with x, w, bias and y one element off 16-byte alignment (its
    output then goes element by element) meets the parity bar, and two calls
    on aligned operands write the same bits."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co, KH, KW, s, p, d = ("c3-5x5-s2", 2, 3, 30, 33, 64, 5, 5, 2, 2, 1)
    L = Layer(name, N, C, H, W, Co, KH, KW, s, p, d, seed=85)
    x, w, b = make_inputs(L, dtype, layout)
    _say(f"[gpu] patch misaligned/twice {dtype} {layout}")
    Ho = oracle.out_size(H, KH, s, p, d)
    Wo = oracle.out_size(W, KW, s, p, d)
    shape = (N, Co, Ho, Wo) if layout == "NCHW" else (N, Ho, Wo, Co)
    y = _misaligned_copy(torch.zeros(shape, dtype=x.dtype))
    cl.conv2d_fwd(_misaligned_copy(x), _misaligned_copy(w), _misaligned_copy(b), s, p, d, layout, "patch", out=y)
    torch.cuda.synchronize()
    xn, wn, bn = make_inputs(L, dtype, "NCHW")
    y_ref, dn = oracle.conv2d(xn, wn, bn, s, p, d, oracle.NCHW)
    _assert_parity(_to_nchw(y, layout), y_ref, dn, dtype, f"patch misaligned {dtype} {layout}")
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    y1 = cl.conv2d_fwd(xd, wd, bd, s, p, d, layout, "patch")
    y2 = cl.conv2d_fwd(xd, wd, bd, s, p, d, layout, "patch")
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16 if dtype == "bf16" else torch.int32),
                       y2.view(torch.int16 if dtype == "bf16" else torch.int32))


# --- edge cases ----------------------------------------------------------------

EDGE = [
    # name, N, C, H, W, Co, KH, KW, s, p, d
    ("1x1-image", 3, 5, 1, 1, 7, 1, 1, 1, 0, 1),
    ("all-padding-rows", 2, 3, 2, 2, 5, 1, 1, 1, 3, 1),
    ("kernel-over-padded-input", 2, 4, 3, 3, 6, 5, 5, 1, 1, 1),
    ("1x1-stride2", 2, 16, 9, 9, 24, 1, 1, 2, 0, 1),
    ("wide-dilation", 1, 8, 20, 17, 9, 3, 3, 1, 5, 4),
    ("tall-kernel", 2, 6, 12, 5, 10, 5, 1, 1, 2, 1),
    ("tiny-K", 3, 1, 7, 7, 3, 1, 2, 1, 0, 1),
    ("odd-everything", 3, 13, 11, 9, 33, 3, 2, 2, 1, 2),
    ("Co-1", 2, 8, 10, 10, 1, 3, 3, 1, 1, 1),
    ("many-channels-skinny", 2, 300, 3, 3, 40, 3, 3, 1, 0, 1),
    ("C-multiple-of-8", 2, 24, 13, 15, 130, 3, 3, 1, 1, 1),
    ("channels-last-copy", 3, 16, 8, 12, 20, 3, 3, 1, 1, 1),     # NCHW copied channels-last, ragged tiles
    ("channels-last-copy-wide", 2, 72, 16, 10, 40, 3, 3, 2, 1, 1),
    # 256 x 128 main loops with output planes whose pixel count is odd, or 2
    # or 4 modulo 8 (NCHW stores in pieces that never cross an image)
    ("planes-odd", 3, 64, 7, 9, 96, 3, 3, 1, 1, 1),
    ("planes-2-mod-8", 4, 32, 9, 10, 130, 3, 3, 1, 1, 1),
    ("planes-4-mod-8", 3, 64, 10, 10, 128, 3, 3, 1, 1, 1),
    # NCHW 1x1 in two parts of the batch (odd N), odd planes
    ("1x1-batch-halves", 3, 16, 7, 9, 24, 1, 1, 1, 0, 1),
    ("1x1-batch-halves-wide", 5, 64, 6, 6, 200, 1, 1, 1, 0, 1),
    # fewer channels than one 16-byte chunk and more than 12 taps: the window
    # tensor padded to one chunk per cell (AUTO and IM2WIN; the stem in both
    # dtypes, the others in fp32 where the padded tensor is below im2col)
    ("small-C-7x7-stem", 4, 3, 40, 40, 40, 7, 7, 2, 3, 1),
    ("small-C-5x5-dilated", 3, 2, 23, 19, 70, 5, 5, 1, 4, 2),
    ("small-C-ragged-Co", 5, 3, 21, 35, 129, 7, 7, 2, 3, 1),
    # channels padded to the next whole 16-byte chunk, several chunks a tap:
    # through the indirection buffer (at most 12 taps) and the window tensor
    ("C-37-3x3", 2, 37, 13, 11, 70, 3, 3, 1, 1, 1),
    ("C-9-3x3", 2, 9, 17, 15, 33, 3, 3, 1, 1, 1),
    ("C-20-5x5-dilated", 3, 20, 23, 19, 50, 5, 5, 2, 4, 2),
    # window rows in LDS: tiles crossing output rows and images, the
    # narrowest output served (a tile starting at column 8 of a 9-wide row
    # spans 30 rows), ragged channels, unpadded kernels
    ("rowwin-narrow", 10, 32, 9, 9, 70, 3, 3, 1, 1, 1),
    ("rowwin-unpadded", 2, 64, 15, 17, 130, 3, 3, 1, 0, 1),
    ("rowwin-tall-kernel", 2, 32, 12, 11, 40, 5, 3, 1, 2, 1),
]


@pytest.mark.parametrize("case", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("algo", ["auto", "indirect", "im2win", "im2col", "direct", "im2win_lds", "patch"])
def test_edge_cases(case, dtype, layout, algo):
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co, KH, KW, s, p, d = case
    L = Layer(name, N, C, H, W, Co, KH, KW, s, p, d, seed=77)
    if algo == "im2win_lds" and not _rowwin_eligible(L, dtype):
        pytest.skip("shape outside the window-rows-in-LDS loop (refused on the host; CPU-tested)")
    if algo == "patch":
        try:
            cl.workspace_size(N, C, H, W, Co, KH, KW, s, p, d, layout, dtype, "patch")
        except cl.ConvLowerError:
            pytest.skip("shape outside PATCH (more than 4 input channels or too many taps; refused on the host)")
    y = _run(L, dtype, layout, algo, N)
    x, w, b = make_inputs(L, dtype, "NCHW")
    y_ref, dn = oracle.conv2d(x, w, b, s, p, d, oracle.NCHW)
    _assert_parity(_to_nchw(y, layout), y_ref, dn, dtype, f"{name} {dtype} {layout} {algo}")


# --- determinism and guard bands ------------------------------------------------

@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("algo", ["auto", "im2win"])
@pytest.mark.parametrize("name", ["C2", "C5c"])
def test_run_twice_bitwise(name, layout, algo):
    L = LAYERS[name]
    x, w, b = make_inputs(L, "bf16", layout, N=4)
    _say(f"[gpu] twice {name} {layout} {algo}")
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    y1 = cl.conv2d_fwd(xd, wd, bd, L.stride, L.pad, L.dilation, layout, algo)
    y2 = cl.conv2d_fwd(xd, wd, bd, L.stride, L.pad, L.dilation, layout, algo)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("algo", ["indirect", "im2win"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_guard_bands(layout, algo, dtype):
    """Nothing is written outside y or outside the queried workspace."""
    L = LAYERS["C5a"]
    n = 2
    x, w, b = make_inputs(L, dtype, layout, N=n)
    _say(f"[gpu] guard {layout} {algo} {dtype}")
    td = x.dtype
    Ho, Wo = cl.output_size(L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation)
    shape = (n, L.Co, Ho, Wo) if layout == "NCHW" else (n, Ho, Wo, L.Co)
    numel = int(np.prod(shape))
    guard = 4096
    ybuf = torch.full((numel + 2 * guard,), 7.0, dtype=td, device=DEV)
    y = ybuf[guard:guard + numel].view(shape)
    need = cl.workspace_size(n, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation, layout, dtype, algo)
    wsbuf = torch.full((need + 4096,), 0xA5, dtype=torch.uint8, device=DEV)
    cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), L.stride, L.pad, L.dilation, layout, algo, out=y,
                  workspace=wsbuf[:need])
    torch.cuda.synchronize()
    assert torch.all(ybuf[:guard] == 7.0) and torch.all(ybuf[guard + numel:] == 7.0)
    assert torch.all(wsbuf[need:] == 0xA5)
    y_ref, dn = _oracle_full(L, dtype, n)
    _assert_parity(_to_nchw(y, layout), y_ref, dn, dtype, "guarded")


# --- the lowering structures themselves ---------------------------------------

GEOMS = [
    # C, H, W, KH, KW, s, p, d
    (64, 56, 56, 3, 3, 1, 1, 1),
    (3, 224, 224, 7, 7, 2, 3, 1),
    (37, 97, 83, 5, 5, 2, 4, 2),
    (5, 9, 7, 2, 3, 3, 2, 1),
]


@pytest.mark.parametrize("geom", GEOMS)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_indirection_buffer_contents(geom, layout):
    C, H, W, KH, KW, s, p, d = geom
    _say(f"[gpu] ibuf {geom} {layout}")
    buf = cl.build_indirection(C, H, W, KH, KW, s, p, d, layout)
    torch.cuda.synchronize()
    ref = oracle.indirection_buffer(H, W, C, KH, KW, s, p, d, oracle.NCHW if layout == "NCHW" else oracle.NHWC)
    assert np.array_equal(buf.cpu().numpy(), ref)


@pytest.mark.parametrize("geom", GEOMS)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_im2win_contents(geom, layout, dtype):
    C, H, W, KH, KW, s, p, d = geom
    g = torch.Generator().manual_seed(3)
    x = torch.randn(2, C, H, W, generator=g).to(torch.float32 if dtype == "fp32" else torch.bfloat16)
    xl = x if layout == "NCHW" else x.permute(0, 2, 3, 1).contiguous()
    _say(f"[gpu] im2win {geom} {layout} {dtype}")
    out = cl.im2win_transform(xl.to(DEV), KH, KW, s, p, d, layout)
    torch.cuda.synchronize()
    ref = oracle.im2win(x, KH, KW, s, p, d, oracle.NCHW)
    assert np.array_equal(out.double().cpu().numpy(), ref)


@pytest.mark.parametrize("geom", GEOMS)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_im2col_contents(geom, layout, dtype):
    """X_col from the HIP transform equals the oracle's plain im2col element
    for element: columns (ci, kh, kw) from NCHW input, (kh, kw, ci) from NHWC."""
    C, H, W, KH, KW, s, p, d = geom
    g = torch.Generator().manual_seed(4)
    x = torch.randn(2, C, H, W, generator=g).to(torch.float32 if dtype == "fp32" else torch.bfloat16)
    xl = x if layout == "NCHW" else x.permute(0, 2, 3, 1).contiguous()
    _say(f"[gpu] im2col {geom} {layout} {dtype}")
    out = cl.im2col_transform(xl.to(DEV), KH, KW, s, p, d, layout)
    torch.cuda.synchronize()
    ref = oracle.im2col(x, KH, KW, s, p, d, oracle.NCHW)
    if layout == "NHWC":
        ref = ref.reshape(-1, C, KH, KW).transpose(0, 2, 3, 1).reshape(ref.shape[0], -1)
    assert np.array_equal(out.double().cpu().numpy(), ref)


# --- the main loop on its own, on operands lowered beforehand -------------------

@pytest.mark.parametrize("algo", ["indirect", "im2win", "im2col"])
@pytest.mark.parametrize("out_layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("name", ["C2", "C5a", "C3e"])
def test_main_loop_entry_matches_full_call(name, algo, out_layout):
    """conv2d_main_loop on a channels-last input (or window tensor), an NHWC
    indirection buffer and OHWI weights gives the same bits as conv2d_fwd.
    Where conv2d_fwd pads the channels to whole 16-byte chunks (C5a through
    the window tensor or the indirection buffer: its K runs over the padded
    channels, so the sums are formed in another order) both are checked
    against the oracle instead."""
    L = LAYERS[name]
    n = 2
    x, w, b = make_inputs(L, "bf16", "NHWC", N=n)
    _say(f"[gpu] main-loop {name} {algo} {out_layout}")
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    y_ref = cl.conv2d_fwd(xd, wd, bd, L.stride, L.pad, L.dilation, "NHWC", algo)
    if algo == "indirect":
        lowered = xd
        ib = cl.build_indirection(L.C, L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation, "NHWC")
    elif algo == "im2col":
        lowered = cl.im2col_transform(xd, L.KH, L.KW, L.stride, L.pad, L.dilation, "NHWC")
        ib = None
    else:
        lowered = cl.im2win_transform(xd, L.KH, L.KW, L.stride, L.pad, L.dilation, "NHWC")
        ib = None
    y = cl.conv2d_main_loop(lowered, ib, wd, bd, None, L.stride, L.pad, L.dilation, algo, out_layout,
                            x_dims=(n, L.C, L.H, L.W))
    torch.cuda.synchronize()
    if out_layout == "NCHW":
        y = y.permute(0, 2, 3, 1)
    padded = L.C % 8 != 0 and (algo == "im2win" or (algo == "indirect" and L.KH * L.KW <= 32 and L.Co <= 64))
    if padded:
        ref, dn = oracle.conv2d(x, w, b, L.stride, L.pad, L.dilation, oracle.NHWC)
        _assert_parity(y.contiguous(), ref, dn, "bf16", f"{name} main loop {out_layout}")
        _assert_parity(y_ref, ref, dn, "bf16", f"{name} full call")
        return
    assert torch.equal(y.contiguous().view(torch.int16), y_ref.view(torch.int16))


# --- main-loop timing stamps ------------------------------------------------------

@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_stamped_main_loop_same_bits_and_inside_the_call(layout):
    """A main loop launched with timing stamps (conv2d_time_next_main_loop)
    writes the same bits as one launched without; its stamped duration is
    positive and no longer than events recorded around the whole call; the
    request covers one launch only."""
    L = LAYERS["C2"]
    x, w, b = make_inputs(L, "bf16", layout, N=4)
    _say(f"[gpu] stamped main loop {layout}")
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    y0 = cl.conv2d_fwd(xd, wd, bd, L.stride, L.pad, L.dilation, layout, "auto")
    ka, kb, ca, cb = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    for e in (ka, kb, ca, cb):
        e.record()
    torch.cuda.synchronize()
    cl.time_next_main_loop(ka, kb)
    ca.record()
    y1 = cl.conv2d_fwd(xd, wd, bd, L.stride, L.pad, L.dilation, layout, "auto")
    cb.record()
    torch.cuda.synchronize()
    k_ms, c_ms = ka.elapsed_time(kb), ca.elapsed_time(cb)
    assert 0 < k_ms <= c_ms, (k_ms, c_ms)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    # consumed: a further call leaves the stamps where they were
    y2 = cl.conv2d_fwd(xd, wd, bd, L.stride, L.pad, L.dilation, layout, "auto")
    torch.cuda.synchronize()
    assert ka.elapsed_time(kb) == k_ms
    assert torch.equal(y0.view(torch.int16), y2.view(torch.int16))


# --- forced main-loop variants (ablation) ---------------------------------------

FORCED_CASES = [
    # name, N, C, H, W, Co, KH, KW, s, p, d
    ("C2-one-image", 1, 64, 56, 56, 128, 3, 3, 1, 1, 1),
    ("planes-odd", 3, 64, 7, 9, 96, 3, 3, 1, 1, 1),
]


@pytest.mark.parametrize("variant", [v for v in cl.MAIN_LOOPS if v != "auto"])
@pytest.mark.parametrize("case", FORCED_CASES, ids=[c[0] for c in FORCED_CASES])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("algo", ["auto", "im2win"])
def test_forced_main_loop_parity(variant, case, dtype, layout, algo):
    """Every main-loop variant, forced, meets the parity bar on the same
    shapes (several tiles and ragged ones, both feeds, both layouts)."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co, KH, KW, s, p, d = case
    L = Layer(name, N, C, H, W, Co, KH, KW, s, p, d, seed=78)
    _say(f"[gpu] forced {variant} {name} {dtype} {layout} {algo}")
    cl.force_main_loop(variant)
    try:
        y = _run(L, dtype, layout, algo, N)
    finally:
        cl.force_main_loop("auto")
    x, w, b = make_inputs(L, dtype, "NCHW")
    y_ref, dn = oracle.conv2d(x, w, b, s, p, d, oracle.NCHW)
    _assert_parity(_to_nchw(y, layout), y_ref, dn, dtype, f"{variant} {name} {dtype} {layout} {algo}")


# --- operands that are element-aligned but not 16-byte aligned -------------------

def _misaligned_copy(t):
    """The same values in a device tensor whose data starts one element past
    an aligned address (so 16-byte vector paths must not be taken)."""
    buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=DEV)
    v = buf[1:1 + t.numel()].view(t.shape)
    v.copy_(t.to(DEV))
    assert v.data_ptr() % 16 != 0
    return v


@pytest.mark.parametrize("case", FORCED_CASES, ids=[c[0] for c in FORCED_CASES])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("algo", ["auto", "indirect", "im2win", "im2win_lds", "im2col", "direct"])
def test_misaligned_operands(case, dtype, layout, algo):
    """x, w, bias and y all one element off 16-byte alignment: every
    algorithm still meets the parity bar (the window-row loop falls back to
    the element-gather loop for NHWC input)."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co, KH, KW, s, p, d = case
    L = Layer(name, N, C, H, W, Co, KH, KW, s, p, d, seed=79)
    x, w, b = make_inputs(L, dtype, layout)
    _say(f"[gpu] misaligned {name} {dtype} {layout} {algo}")
    xd, wd, bd = _misaligned_copy(x), _misaligned_copy(w), _misaligned_copy(b)
    Ho = oracle.out_size(H, KH, s, p, d)
    Wo = oracle.out_size(W, KW, s, p, d)
    shape = (N, Co, Ho, Wo) if layout == "NCHW" else (N, Ho, Wo, Co)
    y = _misaligned_copy(torch.zeros(shape, dtype=x.dtype))
    cl.conv2d_fwd(xd, wd, bd, s, p, d, layout, algo, out=y)
    torch.cuda.synchronize()
    xn, wn, bn = make_inputs(L, dtype, "NCHW")
    y_ref, dn = oracle.conv2d(xn, wn, bn, s, p, d, oracle.NCHW)
    _assert_parity(_to_nchw(y, layout), y_ref, dn, dtype, f"misaligned {name} {dtype} {layout} {algo}")


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_side_stream_parity(layout):
    """conv2d_fwd on a side stream (default priority) that is not torch's
    current stream: the binding allocates the output and workspace on that
    stream, and the result meets the bar."""
    L = LAYERS["C2"]
    x, w, b = make_inputs(L, "bf16", layout, N=4)
    y_ref, dn = _oracle_full(L, "bf16", 4)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = [cl.conv2d_fwd(xd, wd, bd, L.stride, L.pad, L.dilation, layout, "auto", stream=s) for _ in range(3)]
    # work on the current stream meanwhile, allocating and freeing memory
    for _ in range(3):
        t = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
        t.fill_(7)
        del t
    s.synchronize()
    for y in outs:
        _assert_parity(_to_nchw(y, layout), y_ref, dn, "bf16", f"side stream {layout}")


# NCHW 1x1 layers the plain-GEMM feed runs in two half-batch passes, on
# shapes whose few pixels make the plan split K: each pass writes its own
# partial sums and is finished by its own reduce.
SPLIT_1X1 = [((2, 512, 7, 7, 64), "fp32"), ((3, 512, 7, 7, 40), "fp32"), ((5, 512, 14, 14, 96), "fp32"),
             ((4, 1024, 7, 7, 128), "bf16"), ((3, 1024, 7, 7, 40), "bf16"), ((5, 1024, 14, 14, 96), "bf16")]


@pytest.mark.parametrize("shape,dtype", SPLIT_1X1,
                         ids=[f"{s[0]}x{s[1]}x{s[2]}x{s[3]}-{s[4]}-{d}" for s, d in SPLIT_1X1])
@pytest.mark.parametrize("integer", [False, True])
def test_nchw_1x1_halves_with_split_k(shape, dtype, integer):
    from convolution_lowering_amd.workloads import Layer
    N, C, H, W, Co = shape
    L = Layer("split1x1", N, C, H, W, Co, 1, 1, 1, 0, 1, "normal", "normal", 7000 + C, (dtype,))
    ws = cl.workspace_size(N, C, H, W, Co, 1, 1, 1, 0, 1, "NCHW", dtype, "auto")
    copy = ((N + 1) // 2) * C * H * W * (4 if dtype == "fp32" else 2)
    assert ws > copy, "the plan should split K on this shape"
    x, w, b = make_inputs(L, dtype, "NCHW", integer=integer)
    _say(f"[gpu] split 1x1 NCHW {shape} {dtype} integer={integer} workspace={ws}")
    y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), 1, 0, 1, "NCHW", "auto")
    torch.cuda.synchronize()
    y_ref, dn = oracle.conv2d(x, w, b, 1, 0, 1, oracle.NCHW)
    if integer and dtype == "fp32":
        assert np.array_equal(y.double().cpu().numpy(), y_ref)
    else:
        _assert_parity(y, y_ref, dn, dtype, f"split 1x1 {shape}")


# 1x1 NCHW input read where it lies (16-bit types): x[n] is the GEMM's A
# operand transposed, staged in LDS as it lies and turned into MFMA fragments
# by transpose reads.  The four block shapes (128x64 for at most 64 output
# channels, 256x128 with 32- and 64-channel K tiles, 256x256), ragged pixel
# and channel counts, tiles across image boundaries, one image, and split K.
GEMM_NCHW_CASES = [
    # name, N, C, H, W, Co
    ("quad-c3b", 2, 256, 56, 56, 64), ("dual-c3d", 2, 64, 56, 56, 256), ("oct-c5b", 3, 512, 28, 28, 512),
    ("ragged", 3, 32, 6, 20, 40), ("one-image", 1, 64, 16, 24, 128), ("split-k", 2, 1024, 8, 8, 100),
    ("dual-c96", 2, 96, 10, 12, 200), ("oct-sq", 42, 512, 28, 28, 512),
]


@pytest.mark.parametrize("case", GEMM_NCHW_CASES, ids=[c[0] for c in GEMM_NCHW_CASES])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_nchw_1x1_in_place(case, dtype):
    """Against the whole oracle output, to the bar and (integer inputs) to
    the exact result rounded once; the same bits as the channels-last call
    (same tile, same K order); one element off 16-byte alignment, the
    element-gather fallback meets the bar too."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co = case
    L = Layer(name, N, C, H, W, Co, 1, 1, 1, 0, 1, "normal", "kaiming", 9100 + C + Co, (dtype,))
    ws = cl.workspace_size(N, C, H, W, Co, 1, 1, 1, 0, 1, "NCHW", dtype, "auto")
    assert (ws > 0) == (name == "split-k"), f"{name}: workspace {ws}"
    for integer in (False, True):
        x, w, b = make_inputs(L, dtype, "NCHW", integer=integer)
        _say(f"[gpu] in-place 1x1 NCHW {name} {dtype} integer={integer}")
        y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), 1, 0, 1, "NCHW", "auto")
        yn = cl.conv2d_fwd(x.permute(0, 2, 3, 1).contiguous().to(DEV), w.permute(0, 2, 3, 1).contiguous().to(DEV),
                           b.to(DEV), 1, 0, 1, "NHWC", "auto")
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), yn.permute(0, 3, 1, 2).contiguous().view(torch.int16)), name
        y_ref, dn = oracle.conv2d(x, w, b, 1, 0, 1, oracle.NCHW)
        if integer:
            exact = torch.from_numpy(y_ref).float().to(y.dtype).float()
            assert torch.equal(y.float().cpu(), exact), name
        else:
            _assert_parity(y, y_ref, dn, dtype, f"in-place 1x1 NCHW {name}")
    if N * C * H * W <= (1 << 22):
        x, w, b = make_inputs(L, dtype, "NCHW")
        _say(f"[gpu] in-place 1x1 NCHW {name} {dtype} misaligned x")
        xd = _misaligned_copy(x)
        y = cl.conv2d_fwd(xd, w.to(DEV), b.to(DEV), 1, 0, 1, "NCHW", "auto")
        torch.cuda.synchronize()
        y_ref, dn = oracle.conv2d(x, w, b, 1, 0, 1, oracle.NCHW)
        _assert_parity(y, y_ref, dn, dtype, f"in-place 1x1 NCHW {name} misaligned")


# NCHW input read in place by the window-row loop: widths that are and are
# not multiples of the 8-column load (14, 20, 22, 28, 30, 34), padding 0 and 1,
# ragged last tiles, one and several channel slices, 64- and 128-wide tiles.
INPLACE_CASES = [
    ("w56", 2, 64, 56, 56, 128, 1), ("w14", 3, 64, 14, 14, 64, 1), ("w28", 2, 96, 28, 28, 160, 1),
    ("w20", 3, 32, 17, 20, 64, 1), ("w30p0", 2, 32, 21, 30, 128, 0), ("w16", 5, 32, 16, 16, 48, 1),
    ("w112", 1, 32, 112, 112, 64, 1), ("w22", 2, 32, 9, 22, 96, 1), ("w34p0", 2, 32, 11, 34, 64, 0),
]


@pytest.mark.parametrize("case", INPLACE_CASES, ids=[c[0] for c in INPLACE_CASES])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_nchw_window_rows_in_place(case, dtype):
    """The in-place NCHW path meets the bar against the oracle and equals the
    NHWC window-row path bit for bit (same K order, same stage contents);
    integer inputs give the exact result rounded once."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co, p = case
    L = Layer("inplace", N, C, H, W, Co, 3, 3, 1, p, 1, "normal", "normal", 8100 + C + W, (dtype,))
    Ho, Wo = cl.output_size(H, W, 3, 3, 1, p, 1)
    ws = cl.workspace_size(N, C, H, W, Co, 3, 3, 1, p, 1, "NCHW", dtype, "im2win_lds")
    up = lambda v: (v + 255) // 256 * 256
    assert ws == up(Co * C * 9 * 2) + up(Ho * Wo * 9 * 4), f"{name}: expected the in-place plan, workspace {ws}"
    for integer in (False, True):
        x, w, b = make_inputs(L, dtype, "NCHW", integer=integer)
        _say(f"[gpu] in-place NCHW {name} {dtype} integer={integer}")
        y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), 1, p, 1, "NCHW", "im2win_lds")
        xn, wn = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
        yn = cl.conv2d_fwd(xn.to(DEV), wn.to(DEV), b.to(DEV), 1, p, 1, "NHWC", "im2win_lds")
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), yn.permute(0, 3, 1, 2).contiguous().view(torch.int16)), name
        y_ref, dn = oracle.conv2d(x, w, b, 1, p, 1, oracle.NCHW)
        if integer:
            # the exact result (an integer exact in fp32) rounded once
            exact = torch.from_numpy(y_ref).float().to(y.dtype).float()
            assert torch.equal(y.float().cpu(), exact), name
        else:
            _assert_parity(y, y_ref, dn, dtype, f"in-place NCHW {name}")



# --- the ablation loop: each technique switched off, to the same bar --------

ABL_CASES = [
    # name, N, C, H, W, Co, KH, KW, s, p, d
    ("C2-one-image", 1, 64, 56, 56, 128, 3, 3, 1, 1, 1),
    ("ragged", 2, 32, 13, 11, 40, 3, 3, 1, 1, 1),
    ("s2-3x3", 2, 64, 17, 19, 150, 3, 3, 2, 1, 1),
]


@pytest.mark.parametrize("variant", list(cl.ABLATIONS))
@pytest.mark.parametrize("case", ABL_CASES, ids=[c[0] for c in ABL_CASES])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_ablation_loop_parity(variant, case, dtype, layout):
    """Every ablation variant meets the bar against the oracle, and on
    integer inputs gives the exact result rounded once."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co, KH, KW, s, p, d = case
    L = Layer(name, N, C, H, W, Co, KH, KW, s, p, d, seed=91)
    cl.force_main_loop(variant)
    try:
        for integer in (False, True):
            _say(f"[gpu] ablation {variant} {name} {dtype} {layout} integer={integer}")
            y = _run(L, dtype, layout, "auto", N, integer=integer)
            x, w, b = make_inputs(L, dtype, "NCHW", integer=integer)
            y_ref, dn = oracle.conv2d(x, w, b, s, p, d, oracle.NCHW)
            yn = _to_nchw(y, layout)
            if integer:
                exact = torch.from_numpy(y_ref).float().to(y.dtype).float()
                assert torch.equal(yn.float().cpu(), exact), f"{variant} {name} {dtype} {layout}"
            else:
                _assert_parity(yn, y_ref, dn, dtype, f"{variant} {name} {dtype} {layout}")
    finally:
        cl.force_main_loop("auto")



# --- fp8 e4m3 inputs (bf16 bias and output) through the window-row loop ------

FP8_CASES = [
    # name, N, C, H, W, Co
    ("64to128-56", 2, 64, 56, 56, 128), ("128to64-14", 3, 128, 14, 14, 64), ("ragged", 2, 64, 17, 20, 96),
    ("192to256-28", 1, 192, 28, 28, 256),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8_window_rows_nchw(case):
    """NCHW fp8: the channels-last copy and (kh, kw, ci) weights in the
    workspace, then the same loop: the same bits as the NHWC call, and the
    bar against the oracle (integer inputs: the exact result rounded once)."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co = case
    L = Layer(name, N, C, H, W, Co, 3, 3, 1, 1, 1, "normal", "kaiming", 9300 + C, ("fp8",))
    ws = cl.workspace_size(N, C, H, W, Co, 3, 3, 1, 1, 1, "NCHW", "fp8", "auto")
    up = lambda v: (v + 255) // 256 * 256
    assert ws == up(N * C * H * W) + up(Co * C * 9), name
    for integer in (True, False):
        x, w, b = make_inputs(L, "fp8", "NCHW", integer=integer)
        _say(f"[gpu] fp8 NCHW {name} integer={integer}")
        y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), 1, 1, 1, "NCHW", "auto")
        xn, wn = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
        yn = cl.conv2d_fwd(xn.to(DEV), wn.to(DEV), b.to(DEV), 1, 1, 1, "NHWC", "auto")
        torch.cuda.synchronize()
        assert y.dtype == torch.bfloat16
        assert torch.equal(y.view(torch.int16), yn.permute(0, 3, 1, 2).contiguous().view(torch.int16)), name
        y_ref, dn = oracle.conv2d(x, w, b, 1, 1, 1, oracle.NCHW)
        if integer:
            exact = torch.from_numpy(y_ref).float().to(torch.bfloat16).float()
            assert torch.equal(y.float().cpu(), exact), name
        else:
            _assert_parity(y, y_ref, dn, "bf16", f"fp8 NCHW {name}")


@pytest.mark.parametrize("case", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8_window_rows(case):
    """e4m3 x and w, fp32 sums, bf16 y: on integer inputs (exact in e4m3) y is
    the exact result rounded once to bf16; on normal inputs the bf16 bar
    holds against the oracle, which reads the e4m3 values exactly."""
    from convolution_lowering_amd.workloads import Layer
    name, N, C, H, W, Co = case
    L = Layer(name, N, C, H, W, Co, 3, 3, 1, 1, 1, "normal", "kaiming", 9300 + C, ("fp8",))
    for integer in (True, False):
        x, w, b = make_inputs(L, "fp8", "NHWC", integer=integer)
        _say(f"[gpu] fp8 {name} integer={integer}")
        y = cl.conv2d_fwd(x.to(DEV), w.to(DEV), b.to(DEV), 1, 1, 1, "NHWC", "auto")
        torch.cuda.synchronize()
        assert y.dtype == torch.bfloat16
        xr, wr, br = make_inputs(L, "fp8", "NCHW", integer=integer)
        y_ref, dn = oracle.conv2d(xr, wr, br, 1, 1, 1, oracle.NCHW)
        yn = y.permute(0, 3, 1, 2)
        if integer:
            exact = torch.from_numpy(y_ref).float().to(torch.bfloat16).float()
            assert torch.equal(yn.float().cpu(), exact), name
        else:
            _assert_parity(yn, y_ref, dn, "bf16", f"fp8 {name}")
