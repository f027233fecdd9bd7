"""MI355X-native forward convolution lowered onto an MFMA implicit GEMM.

Thin binding over the C ABI of ``include/convlower.h`` (libconvlower.so,
built in-tree by ``convolution_lowering_amd.build``).  Python here only
marshals arguments: it allocates outputs and workspaces with torch, passes
raw device pointers and torch's current HIP stream, and turns status codes
into exceptions.  Every step of the computation runs in the HIP library; if
that library is missing this module raises instead of computing anything
another way.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libconvlower.so")

LAYOUTS = {"NCHW": 0, "NHWC": 1}
ALGOS = {"auto": 0, "indirect": 1, "im2win": 2, "gemm": 3, "im2col": 4, "direct": 5, "im2win_lds": 6, "patch": 7}
DTYPE_CODES = {"fp32": 0, "bf16": 1, "fp16": 2, "fp8": 3}
DTYPE_NAMES = {v: k for k, v in DTYPE_CODES.items()}
STATUS = {0: "CONV_OK", 1: "CONV_ERR_INVALID_ARG", 2: "CONV_ERR_UNSUPPORTED", 3: "CONV_ERR_WORKSPACE",
          4: "CONV_ERR_HIP"}

# Every symbol include/convlower.h declares.
EXPORTS = ("conv_status_string", "conv2d_output_size", "conv2d_fwd_workspace_size", "conv2d_im2col_bytes",
           "conv2d_fwd", "conv2d_main_loop", "conv2d_build_indirection", "conv2d_im2win_transform",
           "conv2d_im2col_transform", "conv2d_force_main_loop", "conv2d_time_next_main_loop",
           "conv2d_fwd_noalloc")
# Size of the per-GPU scratch array conv2d_fwd_noalloc works in
# (CONV_NOALLOC_SCRATCH_BYTES of include/convlower.h).
NOALLOC_SCRATCH_BYTES = 128 << 20
MAIN_LOOPS = {"auto": 0, "element_128x128": 1, "dma_128x128": 2, "dma_256x128": 3, "dual_256x128": 4,
              "oct_256x128": 5, "oct_256x256": 6, "quad_128x64": 7}
# The ablation loop's variants (CONV_MAIN_LOOP_ABL_*): one technique off each.
ABLATIONS = {"abl_full": 8, "abl_no_lds": 9, "abl_one_stage": 10, "abl_no_prefetch": 11, "abl_mfma16": 12,
             "abl_valu": 13, "abl_tile64": 14}


class ConvLowerError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}")
        self.code = code


_lib = None


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m convolution_lowering_amd.build` "
                          "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_size, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    L.conv_status_string.argtypes = [c_int]
    L.conv_status_string.restype = ctypes.c_char_p
    L.conv2d_output_size.argtypes = [c_int] * 7 + [ctypes.POINTER(c_int)] * 2
    L.conv2d_output_size.restype = c_int
    L.conv2d_fwd_workspace_size.argtypes = [c_int] * 13 + [ctypes.POINTER(c_size)]
    L.conv2d_fwd_workspace_size.restype = c_int
    L.conv2d_im2col_bytes.argtypes = [c_int] * 10 + [ctypes.POINTER(c_size)]
    L.conv2d_im2col_bytes.restype = c_int
    L.conv2d_fwd.argtypes = [vp] * 4 + [c_int] * 12 + [vp, vp, c_size, c_int]
    L.conv2d_fwd.restype = c_int
    L.conv2d_fwd_noalloc.argtypes = [vp] * 4 + [c_int] * 12 + [vp, c_int]
    L.conv2d_fwd_noalloc.restype = c_int
    L.conv2d_main_loop.argtypes = [vp] * 5 + [c_int] * 13 + [vp, vp, c_size]
    L.conv2d_main_loop.restype = c_int
    L.conv2d_build_indirection.argtypes = [vp] + [c_int] * 9 + [vp]
    L.conv2d_build_indirection.restype = c_int
    L.conv2d_im2win_transform.argtypes = [vp, vp] + [c_int] * 11 + [vp]
    L.conv2d_im2win_transform.restype = c_int
    L.conv2d_im2col_transform.argtypes = [vp, vp] + [c_int] * 11 + [vp]
    L.conv2d_im2col_transform.restype = c_int
    L.conv2d_force_main_loop.argtypes = [c_int]
    L.conv2d_force_main_loop.restype = c_int
    L.conv2d_time_next_main_loop.argtypes = [vp, vp]
    L.conv2d_time_next_main_loop.restype = c_int
    _lib = L
    return L


def _check(fn, code):
    if code != 0:
        raise ConvLowerError(fn, code)


def _dtype_code(dtype):
    import torch
    if dtype == torch.float32:
        return 0
    if dtype == torch.bfloat16:
        return 1
    if dtype == torch.float16:
        return 2
    if dtype == torch.float8_e4m3fn:
        return 3
    raise TypeError(f"unsupported dtype {dtype}")


def _out_dtype(dtype):
    """Element type of y and bias for inputs of `dtype` (bf16 for fp8)."""
    import torch
    return torch.bfloat16 if dtype == torch.float8_e4m3fn else dtype


def _launch_stream(stream, device):
    """The stream the library launches on: `stream`, else torch's current
    stream on `device`."""
    import torch
    return stream if stream is not None else torch.cuda.current_stream(device)


def _on(stream):
    """Context in which torch allocates on `stream`: a temporary workspace or
    output made there is returned to that stream's pool when freed, so the
    caching allocator cannot hand it to work on another stream while the
    library's kernels on `stream` still use it."""
    import torch
    return torch.cuda.stream(stream)


def output_size(H, W, KH, KW, stride=1, pad=0, dilation=1):
    ho, wo = ctypes.c_int(), ctypes.c_int()
    _check("conv2d_output_size",
           lib().conv2d_output_size(H, W, KH, KW, stride, pad, dilation, ctypes.byref(ho), ctypes.byref(wo)))
    return ho.value, wo.value


def workspace_size(N, C, H, W, Co, KH, KW, stride=1, pad=0, dilation=1, layout="NCHW", dtype="bf16",
                   algo="auto"):
    out = ctypes.c_size_t()
    _check("conv2d_fwd_workspace_size",
           lib().conv2d_fwd_workspace_size(N, C, H, W, Co, KH, KW, stride, pad, dilation, LAYOUTS[layout],
                                           DTYPE_CODES[dtype], ALGOS[algo], ctypes.byref(out)))
    return out.value


def im2col_bytes(N, C, H, W, KH, KW, stride=1, pad=0, dilation=1, dtype="bf16"):
    out = ctypes.c_size_t()
    _check("conv2d_im2col_bytes",
           lib().conv2d_im2col_bytes(N, C, H, W, KH, KW, stride, pad, dilation, DTYPE_CODES[dtype],
                                     ctypes.byref(out)))
    return out.value


def _dims(x, w, layout):
    if layout == "NCHW":
        N, C, H, W = x.shape
        Co, C2, KH, KW = w.shape
    elif layout == "NHWC":
        N, H, W, C = x.shape
        Co, KH, KW, C2 = w.shape
    else:
        raise ValueError(layout)
    if C2 != C:
        raise ValueError("x and w disagree on C_in")
    return N, C, H, W, Co, KH, KW


def _check_tensor(t, name, dtype, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _prepare(x, w, bias, stride, pad, dilation, layout, algo, out, workspace):
    import torch
    N, C, H, W, Co, KH, KW = _dims(x, w, layout)
    dev = x.device
    _check_tensor(x, "x", x.dtype, dev)
    _check_tensor(w, "w", x.dtype, dev)
    ot = _out_dtype(x.dtype)
    if bias is not None:
        _check_tensor(bias, "bias", ot, dev)
        if bias.numel() != Co:
            raise ValueError("bias must hold C_out values")
    dcode = _dtype_code(x.dtype)
    Ho, Wo = output_size(H, W, KH, KW, stride, pad, dilation)
    shape = (N, Co, Ho, Wo) if layout == "NCHW" else (N, Ho, Wo, Co)
    if out is None:
        out = torch.empty(shape, dtype=ot, device=dev)
    else:
        _check_tensor(out, "out", ot, dev)
        if tuple(out.shape) != shape:
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    need = workspace_size(N, C, H, W, Co, KH, KW, stride, pad, dilation, layout, DTYPE_NAMES[dcode], algo)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    dims = (N, C, H, W, Co, KH, KW, stride, pad, dilation, LAYOUTS[layout], dcode)
    return out, dims, ws_ptr, ws_bytes, workspace


def conv2d_fwd(x, w, bias=None, stride=1, pad=0, dilation=1, layout="NCHW", algo="auto", out=None,
               workspace=None, stream=None):
    """y = conv(x, w) + bias on the GPU through conv2d_fwd; returns y.

    x, w, bias, out: contiguous device tensors of one dtype (float32, bfloat16
    or float16) in `layout`; for float8_e4m3fn x and w, bias and out are
    bfloat16.  workspace: optional uint8 device tensor of at
    least workspace_size(...) bytes (allocated here when None)."""
    st = _launch_stream(stream, x.device)
    with _on(st):
        out, dims, ws_ptr, ws_bytes, _ws = _prepare(x, w, bias, stride, pad, dilation, layout, algo, out, workspace)
        code = lib().conv2d_fwd(x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else None,
                                out.data_ptr(), *dims, ctypes.c_void_p(st.cuda_stream), ws_ptr, ws_bytes,
                                ALGOS[algo])
    _check("conv2d_fwd", code)
    return out


def conv2d_fwd_noalloc(x, w, bias, out, stride=1, pad=0, dilation=1, layout="NCHW", algo="auto", stream=None):
    """conv2d_fwd_noalloc: the same convolution as conv2d_fwd into the
    caller's `out`, with the library's per-GPU scratch array as the
    workspace; nothing is allocated on the way (see include/convlower.h)."""
    N, C, H, W, Co, KH, KW = _dims(x, w, layout)
    dev = x.device
    for t, name in ((x, "x"), (w, "w")):
        _check_tensor(t, name, x.dtype, dev)
    _check_tensor(out, "out", _out_dtype(x.dtype), dev)
    if bias is not None:
        _check_tensor(bias, "bias", _out_dtype(x.dtype), dev)
        if bias.numel() != Co:
            raise ValueError("bias must hold C_out values")
    Ho, Wo = output_size(H, W, KH, KW, stride, pad, dilation)
    shape = (N, Co, Ho, Wo) if layout == "NCHW" else (N, Ho, Wo, Co)
    if tuple(out.shape) != shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    st = _launch_stream(stream, dev)
    code = lib().conv2d_fwd_noalloc(x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else None,
                                    out.data_ptr(), N, C, H, W, Co, KH, KW, stride, pad, dilation, LAYOUTS[layout],
                                    _dtype_code(x.dtype), ctypes.c_void_p(st.cuda_stream), ALGOS[algo])
    _check("conv2d_fwd_noalloc", code)
    return out


def conv2d_main_loop(lowered, indirection, w_ohwi, bias, out_shape_nchw, stride=1, pad=0, dilation=1,
                     algo="indirect", out_layout="NCHW", out=None, workspace=None, stream=None, x_dims=None):
    """Steps (c)+(d) on already-lowered operands (see conv2d_main_loop in
    include/convlower.h).  x_dims = (N, C, H, W) of the original input."""
    import torch
    N, C, H, W = x_dims
    Co, KH, KW = w_ohwi.shape[0], w_ohwi.shape[1], w_ohwi.shape[2]
    dev = lowered.device
    _check_tensor(lowered, "lowered", lowered.dtype, dev)
    _check_tensor(w_ohwi, "w_ohwi", lowered.dtype, dev)
    if bias is not None:
        _check_tensor(bias, "bias", lowered.dtype, dev)
    dcode = _dtype_code(lowered.dtype)
    Ho, Wo = output_size(H, W, KH, KW, stride, pad, dilation)
    shape = (N, Co, Ho, Wo) if out_layout == "NCHW" else (N, Ho, Wo, Co)
    st = _launch_stream(stream, dev)
    with _on(st):
        if out is None:
            out = torch.empty(shape, dtype=lowered.dtype, device=dev)
        # The main loop uses only the split-K part of this (for the im2col
        # plan the query also counts X_col itself).
        need = workspace_size(N, C, H, W, Co, KH, KW, stride, pad, dilation, "NHWC", DTYPE_NAMES[dcode], algo)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        code = lib().conv2d_main_loop(lowered.data_ptr(),
                                      indirection.data_ptr() if indirection is not None else None,
                                      w_ohwi.data_ptr(), bias.data_ptr() if bias is not None else None,
                                      out.data_ptr(), N, C, H, W, Co, KH, KW, stride, pad, dilation, ALGOS[algo],
                                      LAYOUTS[out_layout], dcode, ctypes.c_void_p(st.cuda_stream),
                                      workspace.data_ptr() if workspace is not None else None,
                                      workspace.numel() if workspace is not None else 0)
    _check("conv2d_main_loop", code)
    return out


def build_indirection(C, H, W, KH, KW, stride=1, pad=0, dilation=1, layout="NCHW", device="cuda", stream=None):
    """The indirection buffer as an int32 [Ho*Wo, KH*KW] device tensor."""
    import torch
    Ho, Wo = output_size(H, W, KH, KW, stride, pad, dilation)
    st = _launch_stream(stream, torch.device(device))
    with _on(st):
        buf = torch.empty((Ho * Wo, KH * KW), dtype=torch.int32, device=device)
    _check("conv2d_build_indirection",
           lib().conv2d_build_indirection(buf.data_ptr(), C, H, W, KH, KW, stride, pad, dilation,
                                          LAYOUTS[layout], ctypes.c_void_p(st.cuda_stream)))
    return buf


def im2win_transform(x, KH, KW, stride=1, pad=0, dilation=1, layout="NCHW", stream=None):
    """The window-ordered tensor [N][Ho][Wwin][KH][C] as a device tensor."""
    import torch
    if layout == "NCHW":
        N, C, H, W = x.shape
    else:
        N, H, W, C = x.shape
    _check_tensor(x, "x", x.dtype, x.device)
    Ho, Wo = output_size(H, W, KH, KW, stride, pad, dilation)
    Wwin = (Wo - 1) * stride + (KW - 1) * dilation + 1
    st = _launch_stream(stream, x.device)
    with _on(st):
        out = torch.empty((N, Ho, Wwin, KH, C), dtype=x.dtype, device=x.device)
    _check("conv2d_im2win_transform",
           lib().conv2d_im2win_transform(x.data_ptr(), out.data_ptr(), N, C, H, W, KH, KW, stride, pad,
                                         dilation, LAYOUTS[layout], _dtype_code(x.dtype),
                                         ctypes.c_void_p(st.cuda_stream)))
    return out


def im2col_transform(x, KH, KW, stride=1, pad=0, dilation=1, layout="NCHW", stream=None):
    """X_col as a [N*Ho*Wo, C*KH*KW] device tensor: columns (ci, kh, kw) for
    NCHW input, (kh, kw, ci) for NHWC input."""
    import torch
    if layout == "NCHW":
        N, C, H, W = x.shape
    else:
        N, H, W, C = x.shape
    _check_tensor(x, "x", x.dtype, x.device)
    Ho, Wo = output_size(H, W, KH, KW, stride, pad, dilation)
    st = _launch_stream(stream, x.device)
    with _on(st):
        out = torch.empty((N * Ho * Wo, C * KH * KW), dtype=x.dtype, device=x.device)
    _check("conv2d_im2col_transform",
           lib().conv2d_im2col_transform(x.data_ptr(), out.data_ptr(), N, C, H, W, KH, KW, stride, pad,
                                         dilation, LAYOUTS[layout], _dtype_code(x.dtype),
                                         ctypes.c_void_p(st.cuda_stream)))
    return out


def force_main_loop(variant="auto"):
    """Force the main-loop variant of this thread's plans (ablation); "auto"
    restores the library's choice (conv2d_force_main_loop)."""
    code = MAIN_LOOPS[variant] if variant in MAIN_LOOPS else ABLATIONS[variant]
    _check("conv2d_force_main_loop", lib().conv2d_force_main_loop(code))


def time_next_main_loop(start, stop):
    """Have the next main-loop kernel this thread launches stamp two
    torch.cuda.Event objects at its own start and end (conv2d_time_next_main_loop).
    The events must already exist on the device: record each once first."""
    def handle(ev):
        if ev is None:
            return None
        h = ev.cuda_event
        if not h:
            raise ValueError("event not created yet: record it once before passing it")
        return h
    _check("conv2d_time_next_main_loop", lib().conv2d_time_next_main_loop(handle(start), handle(stop)))
