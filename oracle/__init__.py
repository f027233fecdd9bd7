"""Oracle for the convolution forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from it: the two share no code.

Contents
--------
* ``conv2d`` / ``conv2d_points`` -- the plain fp64 seven-loop convolution
  (``conv_oracle.c``), following "Unifying Convolutions and GEMM", section 1,
  extended with zero padding, dilation and bias (section 5 of the same page;
  The Indirect Convolution Algorithm, abstract).  Returns the output and the
  error normaliser  D = sum |x||w| + |bias|.
* ``out_size`` -- the output extent, (in + 2p - d(k-1) - 1) // s + 1
  ("Unifying Convolutions and GEMM", section 5, with the dilation term).
* ``im2col`` -- the unrolled input matrix X_col of shape
  (N*Ho*Wo) x (C*KH*KW) ("Unifying Convolutions and GEMM", section 2).
* ``indirection_buffer`` -- the reading taken of the indirection buffer of
  The Indirect Convolution Algorithm (abstract): one entry per (output pixel,
  kernel tap) holding the element offset of input pixel (hi, wi) of image 0,
  channel 0, or -1 where the tap falls in the zero padding.
* ``im2win`` -- the reading taken of the window-ordered layout of
  "Im2win: An Efficient Convolution Paradigm on GPU" (abstract): for every
  image n and output row ho, the KH input rows that row's windows touch,
  interleaved column by column, channels innermost:
  ``Xwin[n][ho][c][kh][ci] = xpad(n, ci, ho*s + kh*d - p, c - p)`` for
  ``c < Wwin = (Wo-1)*s + (KW-1)*d + 1``.

Pins (tests/test_oracle_*.py): hand-worked 7-loop cases under tests/golden/,
the output-size formula against a brute-force count of window placements,
1x1 stride-1 == plain matrix product, kernel == whole input == dense layer,
NHWC == permuted NCHW, and agreement with torch's own fp64 conv2d and with
the unfold + matmul route.  ``indirection_buffer`` and ``im2win`` are the
pages' structures under a reading of ours (the pages print no example); they
are pinned only through the identity that gathering X_col through them and
multiplying by W_row reproduces the pinned convolution.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

NCHW = 0
NHWC = 1


def build() -> str:
    """Compile conv_oracle.c with gcc (fp64, OpenMP, no FP contraction)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    i32p = ctypes.POINTER(ctypes.c_int32)
    ci = ctypes.c_int
    lib.oracle_out_size.argtypes = [ci] * 5
    lib.oracle_out_size.restype = ci
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ci
    lib.oracle_conv2d_f64.argtypes = [dp, dp, dp, dp, dp] + [ci] * 11
    lib.oracle_conv2d_f64.restype = ci
    lib.oracle_conv2d_points_f64.argtypes = [dp, dp, dp, i32p, ctypes.c_long, dp, dp] + [ci] * 11
    lib.oracle_conv2d_points_f64.restype = ci
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def out_size(n_in: int, k: int, s: int, p: int, d: int) -> int:
    """Number of window placements along one axis (0 if none fits)."""
    span = n_in + 2 * p - d * (k - 1) - 1
    return 0 if span < 0 else span // s + 1


def _as_f64(a):
    """Exact upcast of a numpy array or (CPU) torch tensor to contiguous fp64."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: bf16/fp32 -> fp64 is exact
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, typ=ctypes.c_double):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(typ))


def _dims(x, w, layout):
    if layout == NCHW:
        N, C, H, W = x.shape
        Co, C2, KH, KW = w.shape
    else:
        N, H, W, C = x.shape
        Co, KH, KW, C2 = w.shape
    if C2 != C:
        raise ValueError("channel mismatch between x and w")
    return N, C, H, W, Co, KH, KW


def conv2d(x, w, b=None, stride=1, pad=0, dilation=1, layout=NCHW, want_norm=True):
    """Full fp64 output (and normaliser D) of the seven-loop definition."""
    x, w, b = _as_f64(x), _as_f64(w), _as_f64(b)
    N, C, H, W, Co, KH, KW = _dims(x, w, layout)
    Ho, Wo = out_size(H, KH, stride, pad, dilation), out_size(W, KW, stride, pad, dilation)
    if Ho <= 0 or Wo <= 0:
        raise ValueError("no output placement fits")
    shape = (N, Co, Ho, Wo) if layout == NCHW else (N, Ho, Wo, Co)
    y = np.empty(shape, np.float64)
    dn = np.empty(shape, np.float64) if want_norm else None
    rc = _load().oracle_conv2d_f64(_ptr(x), _ptr(w), _ptr(b), _ptr(y), _ptr(dn),
                                   N, C, H, W, Co, KH, KW, stride, pad, dilation, layout)
    if rc != 0:
        raise RuntimeError(f"oracle_conv2d_f64 failed: {rc}")
    return (y, dn) if want_norm else y


def conv2d_points(x, w, b, pts, stride=1, pad=0, dilation=1, layout=NCHW):
    """fp64 outputs and normalisers at logical points pts[i] = (n, co, ho, wo)."""
    x, w, b = _as_f64(x), _as_f64(w), _as_f64(b)
    N, C, H, W, Co, KH, KW = _dims(x, w, layout)
    pts = np.ascontiguousarray(pts, dtype=np.int32).reshape(-1, 4)
    y = np.empty(len(pts), np.float64)
    dn = np.empty(len(pts), np.float64)
    rc = _load().oracle_conv2d_points_f64(_ptr(x), _ptr(w), _ptr(b), _ptr(pts, ctypes.c_int32),
                                          len(pts), _ptr(y), _ptr(dn),
                                          N, C, H, W, Co, KH, KW, stride, pad, dilation, layout)
    if rc != 0:
        raise RuntimeError(f"oracle_conv2d_points_f64 failed: {rc}")
    return y, dn


def im2col(x, KH, KW, stride=1, pad=0, dilation=1, layout=NCHW):
    """X_col with rows (n, ho, wo) and columns (ci, kh, kw), in fp64.

    Section 2 of "Unifying Convolutions and GEMM": every patch the kernel
    touches, flattened to a row of length C*KH*KW; zero where it overlaps the
    padding.  Plain loops over the patch positions."""
    x = _as_f64(x)
    if layout == NHWC:
        x = np.ascontiguousarray(x.transpose(0, 3, 1, 2))
    N, C, H, W = x.shape
    Ho, Wo = out_size(H, KH, stride, pad, dilation), out_size(W, KW, stride, pad, dilation)
    xp = np.zeros((N, C, H + 2 * pad, W + 2 * pad))
    xp[:, :, pad:pad + H, pad:pad + W] = x
    cols = np.empty((N, Ho, Wo, C, KH, KW))
    for kh in range(KH):
        for kw in range(KW):
            r0, c0 = kh * dilation, kw * dilation
            patch = xp[:, :, r0:r0 + (Ho - 1) * stride + 1:stride, c0:c0 + (Wo - 1) * stride + 1:stride]
            cols[:, :, :, :, kh, kw] = patch.transpose(0, 2, 3, 1)
    return cols.reshape(N * Ho * Wo, C * KH * KW)


def indirection_buffer(H, W, C, KH, KW, stride=1, pad=0, dilation=1, layout=NCHW):
    """int32 [Ho*Wo][KH*KW]: element offset of input pixel (hi, wi) of image 0
    and channel 0 for output pixel p = ho*Wo + wo and tap t = kh*KW + kw, or -1
    where the tap lies in the padding.  NCHW offset hi*W + wi; NHWC offset
    (hi*W + wi)*C (the start of that pixel's row of C channels)."""
    Ho, Wo = out_size(H, KH, stride, pad, dilation), out_size(W, KW, stride, pad, dilation)
    buf = np.empty((Ho * Wo, KH * KW), np.int32)
    for ho in range(Ho):
        for wo in range(Wo):
            for kh in range(KH):
                for kw in range(KW):
                    hi = ho * stride + kh * dilation - pad
                    wi = wo * stride + kw * dilation - pad
                    if 0 <= hi < H and 0 <= wi < W:
                        off = hi * W + wi
                        if layout == NHWC:
                            off *= C
                    else:
                        off = -1
                    buf[ho * Wo + wo, kh * KW + kw] = off
    return buf


def im2win_width(W, KW, stride=1, pad=0, dilation=1):
    """Columns of the padded input that some window touches."""
    Wo = out_size(W, KW, stride, pad, dilation)
    return (Wo - 1) * stride + (KW - 1) * dilation + 1


def im2win(x, KH, KW, stride=1, pad=0, dilation=1, layout=NCHW):
    """The window-ordered tensor Xwin[n][ho][c][kh][ci] in fp64 (see module doc)."""
    x = _as_f64(x)
    if layout == NHWC:
        x = np.ascontiguousarray(x.transpose(0, 3, 1, 2))
    N, C, H, W = x.shape
    Ho = out_size(H, KH, stride, pad, dilation)
    Wwin = im2win_width(W, KW, stride, pad, dilation)
    out = np.zeros((N, Ho, Wwin, KH, C))
    for ho in range(Ho):
        for kh in range(KH):
            hi = ho * stride + kh * dilation - pad
            if not 0 <= hi < H:
                continue
            for c in range(Wwin):
                wi = c - pad
                if 0 <= wi < W:
                    out[:, ho, c, kh, :] = x[:, :, hi, wi]
    return out


def window_from_im2win(xwin, n, ho, wo, KW, stride=1, dilation=1):
    """The (kh, kw, ci) window of output pixel (n, ho, wo) read from Xwin."""
    cols = [wo * stride + kw * dilation for kw in range(KW)]
    blk = xwin[n, ho, cols, :, :]          # [KW][KH][C]
    return blk.transpose(1, 0, 2)           # [KH][KW][C]
