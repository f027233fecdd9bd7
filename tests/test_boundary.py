"""Host-side checks of the C ABI (no GPU needed: nothing here launches a kernel).

The library must load, export every function include/convlower.h declares,
size workspaces below the im2col footprint, and reject bad calls with the
documented status codes before touching the device.
"""
import ctypes
import os
import re

import pytest

import convolution_lowering_amd as cl
import oracle
from convolution_lowering_amd.workloads import LAYERS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convlower.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(conv\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) == 12, names
    L = cl.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(cl.EXPORTS) == names


def test_status_strings():
    L = cl.lib()
    for code, name in cl.STATUS.items():
        assert L.conv_status_string(code).decode() == name


@pytest.mark.parametrize("name", sorted(LAYERS))
def test_output_size_matches_oracle(name):
    L = LAYERS[name]
    ho, wo = cl.output_size(L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation)
    assert ho == oracle.out_size(L.H, L.KH, L.stride, L.pad, L.dilation)
    assert wo == oracle.out_size(L.W, L.KW, L.stride, L.pad, L.dilation)


def _args(L, layout="NCHW", dtype="bf16", algo="auto"):
    return (L.N, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation, layout, dtype, algo)


def _patch_eligible(L, dtype, Wo):
    """The small-input-channel kernel applies: C_in <= 4, the weights of all
    K steps fit its registers (16 steps of 4 taps for 16-bit types, of 2 for
    fp32), and one output row's staged input rows fit 24 KB."""
    es = 4 if dtype == "fp32" else 2
    tps = 2 if dtype == "fp32" else 4
    if L.C > 4 or -(-(L.KH * L.KW) // tps) > 16:
        return False
    win = (Wo - 1) * L.stride + (L.KW - 1) * L.dilation + 1
    rin = (L.KH - 1) * L.dilation + 1
    return rin * win * 4 * es <= 24576


@pytest.mark.parametrize("name", sorted(LAYERS))
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_workspace_below_im2col(name, layout, dtype):
    L = LAYERS[name]
    im2col = cl.im2col_bytes(L.N, L.C, L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation, dtype)
    Ho, Wo = cl.output_size(L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation)
    assert im2col == L.N * Ho * Wo * L.C * L.KH * L.KW * (4 if dtype == "fp32" else 2)
    plain_gemm = (L.KH == L.KW == 1 and L.stride == 1 and L.pad == 0) or (L.KH == L.H and L.KW == L.W and L.pad == 0)
    auto = cl.workspace_size(*_args(L, layout, dtype, "auto"))
    assert auto < im2col
    ind = cl.workspace_size(*_args(L, layout, dtype, "indirect"))
    assert ind < im2col
    if not plain_gemm:
        win = cl.workspace_size(*_args(L, layout, dtype, "im2win"))
        assert win < im2col
        # channels not a whole number of 16-byte chunks with more taps than
        # the indirection feed's LDS slice holds (12; 32 for at most 64
        # output channels): AUTO takes the window tensor with cells padded to
        # whole chunks
        es = 4 if dtype == "fp32" else 2
        T = L.KH * L.KW
        slice_ok = T <= 12 or (T <= 32 and L.Co <= 64 and L.N * Ho * Wo > 64)
        padded_win = (L.C * es) % 16 != 0 and not slice_ok
        # the window rows in LDS where they apply, with more than 64 output
        # channels and at least 256 tiles of 256 x 128
        M = L.N * Ho * Wo
        bn = 64 if L.Co <= 64 else 128  # the window-row tile's width
        rowwin = _rowwin_eligible(L, dtype) and -(-M // 256) * -(-L.Co // bn) >= 256
        if _patch_eligible(L, dtype, Wo):
            assert auto == 0 == cl.workspace_size(*_args(L, layout, dtype, "patch"))
        elif rowwin:
            assert auto == cl.workspace_size(*_args(L, layout, dtype, "im2win_lds"))
        else:
            assert auto == (win if padded_win else ind)
    else:
        # 1x1 NHWC: no workspace at all; 1x1 NCHW: read in place for 16-bit
        # types with C a multiple of 32 and H*W of 8, else the channels-last
        # copy of half the batch; whole-input kernel: only the split-K partials
        whole = L.KH == L.H and L.KW == L.W
        if not whole:
            es = 4 if dtype == "fp32" else 2
            half = (L.N + 1) // 2 * L.C * L.H * L.W * es
            if layout == "NHWC" or _gemm_nchw_eligible(L, dtype):
                assert auto == 0
            else:
                assert auto == (half + 255) // 256 * 256
        assert cl.workspace_size(*_args(L, layout, dtype, "gemm")) == auto


def _gemm_nchw_eligible(L, dtype):
    """The 1x1 NCHW input read where it lies: 16-bit types, C a multiple of
    32, H*W of 8, more than 64 output pixels."""
    return (dtype != "fp32" and L.C % 32 == 0 and (L.H * L.W) % 8 == 0 and L.N * L.H * L.W > 64)


@pytest.mark.parametrize("name", ["C3b", "C3d", "C5b"])
def test_auto_workspace_on_1x1(name):
    """NHWC 1x1 reads x as the GEMM operand in place, and so does NCHW 1x1
    in 16-bit types (x[n] is the operand transposed); fp32 NCHW 1x1 copies
    half the batch at a time channels-last (half of the im2col footprint,
    which for 1x1 is |x|); a single fp32 NCHW image stays on the
    element-gather NCHW feed."""
    L = LAYERS[name]
    for dt in ("bf16", "fp16"):
        assert cl.workspace_size(*_args(L, "NHWC", dt, "auto")) == 0
        assert cl.workspace_size(*_args(L, "NHWC", dt, "gemm")) == 0
        assert cl.workspace_size(*_args(L, "NCHW", dt, "auto")) == 0
        assert cl.workspace_size(*_args(L, "NCHW", dt, "gemm")) == 0
    im2col = cl.im2col_bytes(L.N, L.C, L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation, "fp32")
    ws = cl.workspace_size(*_args(L, "NCHW", "fp32", "auto"))
    assert 0 < ws <= (im2col // 2 + 255) // 256 * 256 < im2col
    one = L.with_batch(1)
    assert cl.workspace_size(*_args(one, "NCHW", "fp32", "auto")) == 0


@pytest.mark.parametrize("shape,dtype,split", [
    ((2, 1024, 8, 8, 100), "bf16", True), ((2, 1024, 8, 8, 100), "fp16", True),
    ((3, 32, 6, 20, 40), "bf16", False), ((1, 64, 16, 24, 128), "fp16", False),
    ((1, 64, 8, 8, 128), "bf16", None),   # 64 pixels: the half-batch/element forms
    ((2, 48, 8, 8, 64), "bf16", None),    # C not a multiple of 32
    ((2, 64, 7, 7, 64), "bf16", None),    # H*W not a multiple of 8
])
def test_nchw_1x1_in_place_plan(shape, dtype, split):
    """The in-place 1x1 NCHW plan: no workspace, or only split-K partials
    where few tiles leave CUs idle (split=True); shapes outside it keep the
    half-batch copy or the element-gather feed (split=None)."""
    N, C, H, W, Co = shape
    ws = cl.workspace_size(N, C, H, W, Co, 1, 1, 1, 0, 1, "NCHW", dtype, "auto")
    if split is None:
        half = ((N + 1) // 2) * C * H * W * 2
        assert ws == 0 if N == 1 else ws >= half
    elif split:
        assert 0 < ws < cl.im2col_bytes(N, C, H, W, 1, 1, 1, 0, 1, dtype)
        assert ws % (N * H * W * Co * 4) == 0  # whole fp32 partial sums, one [M][Co] plane per split
    else:
        assert ws == 0


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("name", ["C3a", "C5a"])
def test_auto_padded_window(name, dtype, layout):
    """The 7x7 stride-2 stem over 3 channels and the dilated 5x5 layer over
    37.  IM2WIN: the window tensor with every (column, kernel row) cell's
    channels padded to whole 16-byte chunks, plus the weights padded to (kh,
    kw, the same channel count).  AUTO: the small-input-channel kernel where
    it applies (the stem in 16-bit types: no workspace); else, for the 25-tap
    5x5 layer with at most 64 output channels, the indirection feed over a
    channels-last copy padded the same way (buffer + copy + weights); else
    the padded window tensor."""
    L = LAYERS[name]
    es = 4 if dtype == "fp32" else 2
    cp = -(-L.C * es // 16) * 16 // es
    Ho, Wo = cl.output_size(L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation)
    Wwin = (Wo - 1) * L.stride + (L.KW - 1) * L.dilation + 1
    up = lambda v: (v + 255) // 256 * 256
    T = L.KH * L.KW
    want = up(L.N * Ho * Wwin * L.KH * cp * es) + up(L.Co * T * cp * es)
    assert cl.workspace_size(*_args(L, layout, dtype, "im2win")) == want
    auto = cl.workspace_size(*_args(L, layout, dtype, "auto"))
    if _patch_eligible(L, dtype, Wo):
        assert auto == 0
    elif T <= 32 and L.Co <= 64:
        ind = up(Ho * Wo * T * 4) + up(L.N * L.H * L.W * cp * es) + up(L.Co * T * cp * es)
        assert auto == cl.workspace_size(*_args(L, layout, dtype, "indirect"))
        assert auto == ind
        assert auto < cl.im2col_bytes(L.N, L.C, L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation, dtype)
    else:
        assert auto == want


@pytest.mark.parametrize("name", sorted(LAYERS))
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_im2col_baseline_workspace_is_x_col(name, layout, dtype):
    """The materialised-im2col baseline holds X_col itself: its workspace is
    the im2col footprint (256-byte aligned), plus split-K partials of at
    most another footprint on skinny layers (the dense C5c layer)."""
    L = LAYERS[name]
    im2col = cl.im2col_bytes(L.N, L.C, L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation, dtype)
    up = (im2col + 255) // 256 * 256
    ws = cl.workspace_size(*_args(L, layout, dtype, "im2col"))
    if name == "C5c":
        assert up < ws <= 2 * up
    else:
        assert ws == up


@pytest.mark.parametrize("name", sorted(LAYERS))
def test_direct_baseline_needs_no_workspace(name):
    L = LAYERS[name]
    for layout in ("NCHW", "NHWC"):
        for dtype in ("fp32", "bf16"):
            assert cl.workspace_size(*_args(L, layout, dtype, "direct")) == 0


def test_main_loop_rejects_direct_and_gemm():
    """conv2d_main_loop takes lowered operands; the direct baseline and the
    plain-GEMM algorithm have none, and are refused on the host."""
    L = cl.lib()
    for algo in (cl.ALGOS["direct"], cl.ALGOS["gemm"], cl.ALGOS["auto"]):
        rc = L.conv2d_main_loop(8, 16, 16, None, 32, 2, 4, 8, 8, 4, 3, 3, 1, 1, 1, algo, 0, 1, None, None, 0)
        assert rc == INVALID


def test_forced_main_loop_checks_on_the_host():
    """A forced main-loop variant the feed cannot serve is refused by the
    query; an unknown variant is an invalid argument; "auto" restores the
    library's choice (the workspace query agrees with it again)."""
    L = LAYERS["C2"]
    auto = cl.workspace_size(*_args(L, "NHWC", "bf16", "auto"))
    odd = cl.workspace_size(24, 24, 13, 15, 130, 3, 3, 1, 1, 1, "NHWC", "bf16", "indirect")
    try:
        for v in cl.MAIN_LOOPS:
            cl.force_main_loop(v)
            assert cl.workspace_size(*_args(L, "NHWC", "bf16", "auto")) >= 0  # C2 takes every variant
        cl.force_main_loop("dual_256x128")  # K tiles would straddle taps at C = 24
        with pytest.raises(cl.ConvLowerError) as e:
            cl.workspace_size(24, 24, 13, 15, 130, 3, 3, 1, 1, 1, "NHWC", "bf16", "indirect")
        assert e.value.code == UNSUPPORTED
        cl.force_main_loop("element_128x128")
        assert cl.workspace_size(24, 24, 13, 15, 130, 3, 3, 1, 1, 1, "NHWC", "bf16", "indirect") >= 0
        assert cl.lib().conv2d_force_main_loop(15) == INVALID
        assert cl.lib().conv2d_force_main_loop(-1) == INVALID
    finally:
        cl.force_main_loop("auto")
    assert cl.workspace_size(*_args(L, "NHWC", "bf16", "auto")) == auto
    assert cl.workspace_size(24, 24, 13, 15, 130, 3, 3, 1, 1, 1, "NHWC", "bf16", "indirect") == odd


def _rowwin_eligible(L, dtype):
    Ho, Wo = cl.output_size(L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation)
    return (L.stride == 1 and L.dilation == 1 and L.KW == 3 and L.C % (16 if dtype == "fp32" else 32) == 0
            and 255 // Wo + 2 <= 32)


@pytest.mark.parametrize("name", sorted(LAYERS))
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_window_rows_in_lds_eligibility_and_workspace(name, dtype):
    """IM2WIN_LDS serves stride-1, dilation-1, three-tap-wide kernels over
    whole channel slices and refuses the rest on the host.  Its workspace is
    the channels-last copy plus OHWI weights for NCHW, and only a spare
    indirection buffer for NHWC."""
    L = LAYERS[name]
    es = 4 if dtype == "fp32" else 2
    up = lambda v: (v + 255) // 256 * 256
    if not _rowwin_eligible(L, dtype):
        for layout in ("NCHW", "NHWC"):
            with pytest.raises(cl.ConvLowerError) as e:
                cl.workspace_size(*_args(L, layout, dtype, "im2win_lds"))
            assert e.value.code == UNSUPPORTED
        return
    Ho, Wo = cl.output_size(L.H, L.W, L.KH, L.KW, L.stride, L.pad, L.dilation)
    ibuf = up(Ho * Wo * L.KH * L.KW * 4)
    assert cl.workspace_size(*_args(L, "NHWC", dtype, "im2win_lds")) == ibuf + _stream_k_bytes(L, Ho, Wo, es, ibuf)
    if dtype != "fp32" and L.W % 2 == 0 and L.Co <= 256 and _raw_runs(L.N * Ho * Wo, Wo, L.W, L.pad) <= 40:
        # NCHW read in place: regrouped weights and a spare indirection buffer
        want = up(L.Co * L.C * L.KH * L.KW * es) + ibuf
    else:
        want = up(L.N * L.C * L.H * L.W * es) + up(L.Co * L.C * L.KH * L.KW * es)
        want += _stream_k_bytes(L, Ho, Wo, es, want)
    assert cl.workspace_size(*_args(L, "NCHW", dtype, "im2win_lds")) == want


@pytest.mark.parametrize("dtype,n,taken", [("bf16", 384, True), ("bf16", 385, False), ("fp16", 384, True),
                                          ("fp16", 385, False), ("fp32", 448, True), ("fp32", 449, False)])
def test_stream_k_taken_up_to_its_tile_bound(dtype, n, taken):
    """3x3 512->128 @16x16, channels-last: N*256 pixels give 192 tiles of
    512 x 128 at N = 384 and 224 at N = 448.  The stream-K form is taken up
    to 3/4 of a tile per block for 16-bit types and 7/8 for fp32, and its
    partial tiles and flags are the last workspace region."""
    ibuf = (16 * 16 * 9 * 4 + 255) // 256 * 256
    sk = (256 * 512 * 128 * 4 + 4 * 256 + 255) // 256 * 256
    ws = cl.workspace_size(n, 512, 16, 16, 128, 3, 3, 1, 1, 1, "NHWC", dtype, "auto")
    assert ws == ibuf + (sk if taken else 0)


def _stream_k_bytes(L, Ho, Wo, es, before):
    """The stream-K region of a channels-last window-row call: 256 partial
    tiles of 512 x 128 fp32 sums and 256 flags, where the layer takes the
    one-block-per-CU form (more than 64 output channels, at least 72 K steps
    of 32 channels (16 for fp32), at most 256 tiles of 512 x 128) with at
    most 3/4 of a tile per block (7/8 for fp32), and the workspace stays
    below im2col."""
    M, K = L.N * Ho * Wo, L.C * L.KH * L.KW
    tiles = -(-M // 512) * -(-L.Co // 128)
    few = tiles * 8 <= 256 * 7 if es == 4 else tiles * 4 <= 256 * 3
    if L.Co <= 64 or K // (16 if es == 4 else 32) < 72 or tiles > 256 or not few:
        return 0
    sk = 256 * 512 * 128 * 4 + 4 * 256
    if before + sk >= M * K * es:
        return 0
    return (sk + 255) // 256 * 256


def _raw_runs(M, Wo, W, p):
    """Runs of 8 in-image input columns (starting at multiples of 8) that the
    busiest 256-pixel tile of a 3-wide window needs per channel: for each
    output row the tile touches, the in-image part of the columns its
    windows cover, counted tile by tile."""
    worst = 0
    for m0 in range(0, M, 256):
        mend = min(m0 + 256, M)
        runs = 0
        for R in range(m0 // Wo, (mend - 1) // Wo + 1):
            first, last = max(m0, R * Wo), min(mend, (R + 1) * Wo)
            lo = first - R * Wo - p
            hi = lo + (last - first) + 2
            lo, hi = max(lo, 0), min(hi, W)
            if hi > lo:
                runs += len(range(lo // 8, (hi - 1) // 8 + 1))
        worst = max(worst, runs)
    return worst


@pytest.mark.parametrize("shape", [(2, 32, 16, 16), (3, 32, 18, 14), (1, 64, 20, 30), (2, 32, 12, 12),
                                   (1, 32, 9, 11), (2, 32, 40, 10)])
def test_nchw_window_rows_read_in_place_where_runs_fit(shape):
    """The in-place NCHW form of the window-row loop (16-bit, even W, at most
    256 output channels, every tile's runs within 40 per channel) needs no
    copy of x; elsewhere the channels-last copy stays."""
    N, C, H, W = shape
    Ho, Wo = cl.output_size(H, W, 3, 3, 1, 1, 1)
    if 255 // Wo + 2 > 32:
        pytest.skip("outside the window-row loop")
    ws = cl.workspace_size(N, C, H, W, 64, 3, 3, 1, 1, 1, "NCHW", "bf16", "im2win_lds")
    up = lambda v: (v + 255) // 256 * 256
    inplace = W % 2 == 0 and _raw_runs(N * Ho * Wo, Wo, W, 1) <= 40
    small = up(64 * C * 9 * 2) + up(Ho * Wo * 9 * 4)
    assert (ws == small) == inplace, (shape, ws, small)


@pytest.mark.parametrize("W,ok", [(7, False), (8, False), (9, True), (10, True)])
def test_window_rows_in_lds_needs_nine_output_columns(W, ok):
    """A 256-pixel tile of the window-row loop may span at most 32 output
    rows: 255 // Wo + 2 of them, so Wo = 9 is the narrowest output served."""
    args = (3, 32, 12, W, 64, 3, 3, 1, 1, 1, "NHWC", "bf16", "im2win_lds")
    if ok:
        assert cl.workspace_size(*args) > 0
    else:
        with pytest.raises(cl.ConvLowerError) as e:
            cl.workspace_size(*args)
        assert e.value.code == UNSUPPORTED


def test_gemm_algo_rejected_on_windowed_layer():
    L = LAYERS["C2"]
    with pytest.raises(cl.ConvLowerError) as e:
        cl.workspace_size(*_args(L, "NCHW", "bf16", "gemm"))
    assert e.value.code == UNSUPPORTED


def test_indirection_workspace_is_the_buffer():
    L = LAYERS["C2"]
    ws = cl.workspace_size(*_args(L, "NHWC", "bf16", "indirect"))
    assert ws == (56 * 56 * 9 * 4 + 255) // 256 * 256


@pytest.mark.parametrize("bad", [
    dict(N=0), dict(C=0), dict(H=0), dict(W=-1), dict(Co=0), dict(KH=0), dict(KW=0),
    dict(s=0), dict(p=-1), dict(d=0), dict(KH=20),  # kernel larger than padded input
])
def test_invalid_sizes(bad):
    a = dict(N=2, C=4, H=8, W=8, Co=4, KH=3, KW=3, s=1, p=1, d=1)
    a.update(bad)
    out = ctypes.c_size_t()
    code = cl.lib().conv2d_fwd_workspace_size(a["N"], a["C"], a["H"], a["W"], a["Co"], a["KH"], a["KW"], a["s"],
                                              a["p"], a["d"], 0, 1, 0, ctypes.byref(out))
    assert code == INVALID


def test_invalid_enums_and_null_outputs():
    L = cl.lib()
    out = ctypes.c_size_t()
    base = (2, 4, 8, 8, 4, 3, 3, 1, 1, 1)
    assert L.conv2d_fwd_workspace_size(*base, 2, 1, 0, ctypes.byref(out)) == INVALID   # layout
    assert L.conv2d_fwd_workspace_size(*base, 0, 7, 0, ctypes.byref(out)) == INVALID   # dtype
    assert L.conv2d_fwd_workspace_size(*base, 0, 1, 9, ctypes.byref(out)) == INVALID   # algo
    assert L.conv2d_fwd_workspace_size(*base, 0, 1, 8, ctypes.byref(out)) == INVALID   # one past PATCH
    assert L.conv2d_fwd_workspace_size(*base, 0, 1, -1, ctypes.byref(out)) == INVALID
    assert L.conv2d_fwd_workspace_size(*base, 0, 1, 0, None) == INVALID


def test_fwd_rejects_before_launch():
    """These return on the host, so they are safe without a GPU."""
    L = cl.lib()
    fake = ctypes.c_void_p(0x1000)
    args = (2, 4, 8, 8, 4, 3, 3, 1, 1, 1, 0, 1, None)
    # NULL x / w / y
    assert L.conv2d_fwd(None, fake, None, fake, *args, fake, 1 << 20, 1) == INVALID
    assert L.conv2d_fwd(fake, None, None, fake, *args, fake, 1 << 20, 1) == INVALID
    assert L.conv2d_fwd(fake, fake, None, None, *args, fake, 1 << 20, 1) == INVALID
    # workspace missing or short (the indirect algo needs one)
    assert L.conv2d_fwd(fake, fake, None, fake, *args, None, 0, 1) == WORKSPACE
    assert L.conv2d_fwd(fake, fake, None, fake, *args, fake, 16, 1) == WORKSPACE
    # misaligned bf16 pointer
    odd = ctypes.c_void_p(0x1001)
    assert L.conv2d_fwd(odd, fake, None, fake, *args, fake, 1 << 20, 1) == INVALID
    # bad geometry
    bad = (2, 4, 8, 8, 4, 30, 3, 1, 1, 1, 0, 1, None)
    assert L.conv2d_fwd(fake, fake, None, fake, *bad, fake, 1 << 20, 1) == INVALID
    assert L.conv2d_build_indirection(None, 4, 8, 8, 3, 3, 1, 1, 1, 0, None) == INVALID
    # the main-loop entry takes only the two lowerings, and needs the buffer for INDIRECT
    assert L.conv2d_main_loop(fake, fake, fake, None, fake, 2, 8, 8, 8, 4, 3, 3, 1, 1, 1, 0, 0, 1, None, fake,
                              1 << 20) == INVALID
    assert L.conv2d_main_loop(fake, None, fake, None, fake, 2, 8, 8, 8, 4, 3, 3, 1, 1, 1, 1, 0, 1, None, fake,
                              1 << 20) == INVALID
    assert L.conv2d_im2win_transform(None, fake, 1, 4, 8, 8, 3, 3, 1, 1, 1, 0, 1, None) == INVALID


def test_oversized_request_is_unsupported():
    out = ctypes.c_size_t()
    code = cl.lib().conv2d_fwd_workspace_size(4096, 512, 512, 512, 64, 3, 3, 1, 1, 1, 0, 1, 0, ctypes.byref(out))
    assert code == UNSUPPORTED


def test_noalloc_rejects_a_workspace_past_the_scratch_array():
    """conv2d_fwd_noalloc refuses, on the host and before any HIP call, a
    plan whose workspace exceeds its scratch array (the im2col baseline on
    the 64->128 layer at 112x112 needs 1.85 GB); bad arguments are still
    INVALID_ARG first."""
    L = cl.lib()
    need = cl.workspace_size(128, 64, 112, 112, 128, 3, 3, 1, 1, 1, "NCHW", "bf16", "im2col")
    assert need > cl.NOALLOC_SCRATCH_BYTES
    args = (128, 64, 112, 112, 128, 3, 3, 1, 1, 1, 0, 1, None, cl.ALGOS["im2col"])
    assert L.conv2d_fwd_noalloc(None, None, None, None, *args) == WORKSPACE
    bad = (128, 64, 112, 112, 128, 3, 3, 0, 1, 1, 0, 1, None, cl.ALGOS["auto"])  # stride 0
    assert L.conv2d_fwd_noalloc(None, None, None, None, *bad) == INVALID


def test_noalloc_drops_the_stream_k_regions_before_refusing():
    """A plan that exceeds the scratch array only by its stream-K partial
    tiles is not refused: fp32 3x3 256->128 @28, NCHW, N = 88 needs 138.9 MB
    with them and 71.8 MB without, so the call gets past the workspace check
    (it then needs the device for the scratch array's address, or stops at
    the null pointers: anything but WORKSPACE)."""
    L = cl.lib()
    need = cl.workspace_size(88, 256, 28, 28, 128, 3, 3, 1, 1, 1, "NCHW", "fp32", "auto")
    sk = 256 * 512 * 128 * 4 + 1024
    assert need > cl.NOALLOC_SCRATCH_BYTES >= need - sk
    args = (88, 256, 28, 28, 128, 3, 3, 1, 1, 1, 0, 0, None, cl.ALGOS["auto"])
    assert L.conv2d_fwd_noalloc(None, None, None, None, *args) in (INVALID, HIP)


@pytest.mark.parametrize("shape,dtype", [((2, 512, 7, 7, 64), "fp32"), ((4, 1024, 7, 7, 128), "bf16")])
def test_nchw_1x1_halves_plan_split_partials(shape, dtype):
    """Late-network 1x1 NCHW shapes: the half-batch copy plus split-K
    partials, all below the im2col footprint (the partials region is the
    one every half-batch pass reuses)."""
    N, C, H, W, Co = shape
    es = 4 if dtype == "fp32" else 2
    ws = cl.workspace_size(N, C, H, W, Co, 1, 1, 1, 0, 1, "NCHW", dtype, "auto")
    copy = ((N + 1) // 2) * C * H * W * es
    assert copy < ws < cl.im2col_bytes(N, C, H, W, 1, 1, 1, 0, 1, dtype)


def test_ablation_loops_plan_on_the_host():
    """The ablation loop's variants run the indirection feed on 16-bit types
    with C_in a multiple of 32: AUTO becomes INDIRECT (the workspace is the
    indirection buffer for NHWC, never split-K partials), fp32, C_in = 24 and
    the window-ordered feed are refused before any launch."""
    L = LAYERS["C2"]
    up = lambda v: (v + 255) // 256 * 256
    ibuf = up(56 * 56 * 9 * 4)
    try:
        for v in cl.ABLATIONS:
            cl.force_main_loop(v)
            assert cl.workspace_size(*_args(L, "NHWC", "bf16", "auto")) == ibuf
            assert cl.workspace_size(*_args(L, "NHWC", "fp16", "indirect")) == ibuf
            # a skinny layer that the other loops split over K
            assert cl.workspace_size(2, 512, 7, 7, 64, 3, 3, 1, 1, 1, "NHWC", "bf16", "auto") == up(49 * 9 * 4)
            for args in ((*_args(L, "NHWC", "fp32", "auto")[:-1], "auto"),
                         (24, 24, 13, 15, 130, 3, 3, 1, 1, 1, "NHWC", "bf16", "indirect"),
                         (*_args(L, "NHWC", "bf16", "im2win")[:-1], "im2win")):
                with pytest.raises(cl.ConvLowerError) as e:
                    cl.workspace_size(*args)
                assert e.value.code == UNSUPPORTED, (v, args)
    finally:
        cl.force_main_loop("auto")


def test_fp8_plans_only_window_rows():
    """fp8 e4m3 inputs run the window-row loop with C_in a multiple of 64:
    channels-last tensors with no workspace, NCHW tensors (H*W a multiple of
    4) with the channels-last copy of x and the regrouped weights (|x| + |w|
    bytes); other algorithms, C_in not a multiple of 64, stride 2, NCHW with
    H*W not a multiple of 4 and the lowering transforms are refused on the
    host."""
    L = LAYERS["C2"]
    up = lambda v: (v + 255) // 256 * 256
    assert cl.workspace_size(*_args(L, "NHWC", "fp8", "auto")) == 0
    assert cl.workspace_size(*_args(L, "NHWC", "fp8", "im2win_lds")) == 0
    assert cl.workspace_size(*_args(L, "NCHW", "fp8", "auto")) == up(L.N * L.C * L.H * L.W) + up(L.Co * L.C * 9)
    for args in (_args(L, "NHWC", "fp8", "indirect"), _args(L, "NCHW", "fp8", "indirect"),
                 _args(L, "NHWC", "fp8", "im2col"), (2, 32, 16, 16, 64, 3, 3, 1, 1, 1, "NHWC", "fp8", "auto"),
                 (2, 64, 16, 16, 64, 3, 3, 2, 1, 1, "NHWC", "fp8", "auto"),
                 (2, 64, 15, 15, 64, 3, 3, 1, 1, 1, "NCHW", "fp8", "auto")):
        with pytest.raises(cl.ConvLowerError) as e:
            cl.workspace_size(*args)
        assert e.value.code == UNSUPPORTED, args
    assert cl.lib().conv2d_im2win_transform(None, None, 1, 64, 8, 8, 3, 3, 1, 1, 1, 1, 3, None) == UNSUPPORTED
    assert cl.lib().conv2d_im2col_transform(None, None, 1, 64, 8, 8, 3, 3, 1, 1, 1, 1, 3, None) == UNSUPPORTED
    assert cl.im2col_bytes(L.N, L.C, L.H, L.W, 3, 3, 1, 1, 1, "fp8") == L.N * 56 * 56 * 64 * 9
