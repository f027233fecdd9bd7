"""Pins of the oracle's lowering structures (im2col, indirection buffer, im2win).

The pages print no example of any of these tensors, so their contents are
pinned only through identities: X_col @ W_row^T + b must reproduce the
seven-loop convolution ("Unifying Convolutions and GEMM", sections 2-3), and
the rows gathered through the indirection buffer or read out of the im2win
tensor must be exactly the rows of X_col.
"""
import numpy as np
import pytest

import oracle
from convolution_lowering_amd.workloads import LAYERS

SHAPES = [
    # N, C, H, W, Co, KH, KW, s, p, d
    (2, 3, 7, 6, 4, 3, 3, 1, 1, 1),
    (1, 2, 9, 9, 3, 3, 2, 2, 2, 2),
    (2, 4, 5, 8, 2, 1, 1, 1, 0, 1),
    (1, 3, 6, 6, 2, 6, 6, 1, 0, 1),
    (1, 2, 11, 10, 3, 5, 5, 2, 4, 2),
    (3, 1, 4, 4, 2, 2, 3, 3, 0, 1),
]


def _data(shape, seed):
    N, C, H, W, Co, KH, KW, s, p, d = shape
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, C, H, W)), rng.standard_normal((Co, C, KH, KW)),
            rng.standard_normal(Co))


@pytest.mark.parametrize("shape", SHAPES)
def test_im2col_gemm_equals_convolution(shape):
    N, C, H, W, Co, KH, KW, s, p, d = shape
    x, w, b = _data(shape, 1)
    cols = oracle.im2col(x, KH, KW, s, p, d)
    Ho, Wo = oracle.out_size(H, KH, s, p, d), oracle.out_size(W, KW, s, p, d)
    assert cols.shape == (N * Ho * Wo, C * KH * KW)
    y_col = cols @ w.reshape(Co, -1).T + b
    y = oracle.conv2d(x, w, b, s, p, d, want_norm=False)
    np.testing.assert_allclose(y_col.reshape(N, Ho, Wo, Co).transpose(0, 3, 1, 2), y,
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("layout", [oracle.NCHW, oracle.NHWC])
def test_indirection_buffer_gathers_im2col(shape, layout):
    N, C, H, W, Co, KH, KW, s, p, d = shape
    x, w, b = _data(shape, 2)
    buf = oracle.indirection_buffer(H, W, C, KH, KW, s, p, d, layout)
    Ho, Wo = oracle.out_size(H, KH, s, p, d), oracle.out_size(W, KW, s, p, d)
    assert buf.shape == (Ho * Wo, KH * KW) and buf.dtype == np.int32
    xl = x if layout == oracle.NCHW else x.transpose(0, 2, 3, 1)
    flat = np.ascontiguousarray(xl).reshape(N, -1)
    gathered = np.zeros((N, Ho * Wo, C, KH * KW))
    for n in range(N):
        for pix in range(Ho * Wo):
            for t in range(KH * KW):
                off = buf[pix, t]
                if off < 0:
                    continue
                for ci in range(C):
                    step = H * W if layout == oracle.NCHW else 1
                    gathered[n, pix, ci, t] = flat[n, off + ci * step]
    cols = oracle.im2col(x, KH, KW, s, p, d)
    assert np.array_equal(gathered.reshape(N * Ho * Wo, -1), cols)
    # every sentinel is a tap in the padding, every other entry lies in the image
    for pix in range(Ho * Wo):
        ho, wo = divmod(pix, Wo)
        for t in range(KH * KW):
            kh, kw = divmod(t, KW)
            hi, wi = ho * s + kh * d - p, wo * s + kw * d - p
            inside = 0 <= hi < H and 0 <= wi < W
            assert (buf[pix, t] >= 0) == inside


@pytest.mark.parametrize("shape", SHAPES)
def test_im2win_windows_are_im2col_rows(shape):
    N, C, H, W, Co, KH, KW, s, p, d = shape
    x, w, b = _data(shape, 3)
    xwin = oracle.im2win(x, KH, KW, s, p, d)
    Ho, Wo = oracle.out_size(H, KH, s, p, d), oracle.out_size(W, KW, s, p, d)
    assert xwin.shape == (N, Ho, oracle.im2win_width(W, KW, s, p, d), KH, C)
    cols = oracle.im2col(x, KH, KW, s, p, d).reshape(N, Ho, Wo, C, KH, KW)
    for n in range(N):
        for ho in range(Ho):
            for wo in range(Wo):
                win = oracle.window_from_im2win(xwin, n, ho, wo, KW, s, d)  # [KH][KW][C]
                assert np.array_equal(win.transpose(2, 0, 1), cols[n, ho, wo])
    # NHWC input gives the same tensor
    xwin2 = oracle.im2win(x.transpose(0, 2, 3, 1), KH, KW, s, p, d, oracle.NHWC)
    assert np.array_equal(xwin, xwin2)


def test_im2win_window_is_contiguous_for_unit_dilation():
    """The window of one output pixel is one contiguous run of KW*KH*C values
    when dilation is 1 -- the continuity the im2win abstract claims."""
    N, C, H, W, KH, KW, s, p = 1, 3, 6, 7, 3, 3, 1, 1
    x = np.arange(N * C * H * W, dtype=np.float64).reshape(N, C, H, W) + 1
    xwin = oracle.im2win(x, KH, KW, s, p, 1)
    flat = xwin.reshape(N, xwin.shape[1], -1)
    for ho in range(xwin.shape[1]):
        for wo in range(oracle.out_size(W, KW, s, p, 1)):
            run = flat[0, ho, wo * s * KH * C: (wo * s + KW) * KH * C]
            win = oracle.window_from_im2win(xwin, 0, ho, wo, KW, s, 1)  # [KH][KW][C]
            assert np.array_equal(np.sort(run), np.sort(win.reshape(-1)))


@pytest.mark.parametrize("name", sorted(LAYERS))
def test_lowering_footprints(name):
    """im2win is below im2col on every layer but the 1x1 / whole-input ones,
    and the indirection buffer is far below both."""
    L = LAYERS[name]
    Ho = oracle.out_size(L.H, L.KH, L.stride, L.pad, L.dilation)
    Wo = oracle.out_size(L.W, L.KW, L.stride, L.pad, L.dilation)
    im2col = L.N * Ho * Wo * L.C * L.KH * L.KW
    win = L.N * Ho * oracle.im2win_width(L.W, L.KW, L.stride, L.pad, L.dilation) * L.KH * L.C
    ind = Ho * Wo * L.KH * L.KW  # int32 entries, shared across the batch
    if L.KH == 1 and L.KW == 1 or (L.KH == L.H and L.KW == L.W):
        assert win == im2col
    else:
        assert win < im2col
    assert ind * 4 < im2col * 2
