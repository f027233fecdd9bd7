"""Layer shapes and seeded synthetic inputs.

This module is shared by the tests, the benchmark and the smoke check: it
only draws inputs and holds the shape table.  It computes nothing of the
convolution itself (not even output sizes), so the oracle and the HIP path
can both be fed from it without sharing any of the method's arithmetic.

Shapes stand in for the unlisted "twelve DNN benchmarks" of "Im2win: An
Efficient Convolution Paradigm on GPU" (abstract): ResNet-50 and VGG-16 shaped
layers (both networks are on that page's reference list), the verification
layer of "Unifying Convolutions and GEMM" (section 5: N=32, C_in=64, 56x56,
C_out=128, 3x3, stride 1, pad 1), and a generality sweep.

Draw recipe (one torch CPU generator per layer, seed = 1000*set + index):
x, then w, then bias, all float32, then cast to the requested dtype with
round-to-nearest-even (for fp8: x and w to e4m3, the bias to bf16).
Distributions: N(0,1) inputs for C1/C2/C3/C5, uniform[-1,1] for C4; N(0,1) weights for C1/C2/C5, Kaiming-normal
(std = sqrt(2 / (C_in*KH*KW))) for C3/C4; bias N(0,1) everywhere.
Values are drawn in the logical NCHW / OIHW order and permuted for NHWC /
OHWI, so both layouts of one layer hold the same numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Layer:
    name: str
    N: int
    C: int
    H: int
    W: int
    Co: int
    KH: int
    KW: int
    stride: int = 1
    pad: int = 0
    dilation: int = 1
    xdist: str = "normal"      # "normal" | "uniform"
    wdist: str = "normal"      # "normal" | "kaiming"
    seed: int = 0
    dtypes: tuple = ("bf16",)
    layouts: tuple = ("NCHW", "NHWC")
    note: str = ""

    @property
    def flops_per_output(self) -> int:
        return 2 * self.C * self.KH * self.KW

    def with_batch(self, n: int) -> "Layer":
        return replace(self, N=n)


def _L(name, N, C, H, W, Co, K, s, p, d, xdist, wdist, seed, dtypes, note, KW=None):
    return Layer(name, N, C, H, W, Co, K, K if KW is None else KW, s, p, d, xdist, wdist, seed,
                 dtypes, ("NCHW", "NHWC"), note)


LAYERS = {
    "C1": _L("C1", 2, 16, 16, 16, 32, 3, 1, 1, 1, "normal", "normal", 1000, ("fp32",),
             "single 3x3 layer, parity case"),
    "C2": _L("C2", 32, 64, 56, 56, 128, 3, 1, 1, 1, "normal", "normal", 2000, ("fp32", "bf16"),
             "3x3 64->128 @56, the blog's verification layer"),
    "C3a": _L("C3a", 64, 3, 224, 224, 64, 7, 2, 3, 1, "normal", "kaiming", 3000, ("bf16",),
              "ResNet-50 stem 7x7 s2 p3 3->64 @224"),
    "C3b": _L("C3b", 64, 256, 56, 56, 64, 1, 1, 0, 1, "normal", "kaiming", 3001, ("bf16",),
              "ResNet-50 bottleneck 1x1 256->64 @56"),
    "C3c": _L("C3c", 64, 64, 56, 56, 64, 3, 1, 1, 1, "normal", "kaiming", 3002, ("bf16",),
              "ResNet-50 bottleneck 3x3 64->64 @56"),
    "C3d": _L("C3d", 64, 64, 56, 56, 256, 1, 1, 0, 1, "normal", "kaiming", 3003, ("bf16",),
              "ResNet-50 bottleneck 1x1 64->256 @56"),
    "C3e": _L("C3e", 64, 128, 56, 56, 128, 3, 2, 1, 1, "normal", "kaiming", 3004, ("bf16",),
              "ResNet-50 3x3 s2 128->128 56->28"),
    "C4a": _L("C4a", 128, 3, 224, 224, 64, 3, 1, 1, 1, "uniform", "kaiming", 4000, ("bf16",),
              "VGG-16 3x3 3->64 @224"),
    "C4b": _L("C4b", 128, 64, 112, 112, 128, 3, 1, 1, 1, "uniform", "kaiming", 4001, ("bf16",),
              "VGG-16 3x3 64->128 @112"),
    "C4c": _L("C4c", 128, 128, 56, 56, 256, 3, 1, 1, 1, "uniform", "kaiming", 4002, ("bf16",),
              "VGG-16 3x3 128->256 @56"),
    "C4d": _L("C4d", 128, 256, 28, 28, 512, 3, 1, 1, 1, "uniform", "kaiming", 4003, ("bf16",),
              "VGG-16 3x3 256->512 @28"),
    "C4e": _L("C4e", 128, 512, 14, 14, 512, 3, 1, 1, 1, "uniform", "kaiming", 4004, ("bf16",),
              "VGG-16 3x3 512->512 @14"),
    "C5a": _L("C5a", 16, 37, 97, 83, 61, 5, 2, 4, 2, "normal", "normal", 5000, ("fp32", "bf16"),
              "5x5 dilation 2 stride 2 pad 4, 37->61 @97x83"),
    "C5b": _L("C5b", 16, 512, 28, 28, 512, 1, 1, 0, 1, "normal", "normal", 5001, ("fp32", "bf16"),
              "1x1 512->512 @28 (a plain GEMM)"),
    "C5c": _L("C5c", 16, 512, 7, 7, 1000, 7, 1, 0, 1, "normal", "normal", 5002, ("fp32", "bf16"),
              "7x7 kernel over a 7x7 input, 512->1000 (a dense layer)"),
}

TORCH_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16, "fp8": torch.float8_e4m3fn}


def make_inputs(layer: Layer, dtype: str = "bf16", layout: str = "NCHW", *, N: int | None = None,
                seed: int | None = None, bias: bool = True, integer: bool = False):
    """Seeded CPU tensors (x, w, b) for one layer, contiguous in `layout`.

    integer=True draws every value from {-3..3}: then each product and every
    partial sum of a layer in this table is an exactly representable float32
    integer, so any correct float32 path reproduces the exact result."""
    n = layer.N if N is None else N
    g = torch.Generator("cpu").manual_seed(layer.seed if seed is None else seed)
    xs = (n, layer.C, layer.H, layer.W)
    ws = (layer.Co, layer.C, layer.KH, layer.KW)
    if integer:
        x = torch.randint(-3, 4, xs, generator=g).float()
        w = torch.randint(-3, 4, ws, generator=g).float()
        b = torch.randint(-3, 4, (layer.Co,), generator=g).float()
    else:
        if layer.xdist == "uniform":
            x = torch.rand(xs, generator=g) * 2.0 - 1.0
        else:
            x = torch.randn(xs, generator=g)
        w = torch.randn(ws, generator=g)
        if layer.wdist == "kaiming":
            w = w * (2.0 / (layer.C * layer.KH * layer.KW)) ** 0.5
        b = torch.randn((layer.Co,), generator=g)
    td = TORCH_DTYPES[dtype]
    # fp8: x and w in e4m3 (torch rounds to nearest even), bias in bf16
    x, w, b = x.to(td), w.to(td), b.to(torch.bfloat16 if dtype == "fp8" else td)
    if layout == "NHWC":
        x = x.permute(0, 2, 3, 1).contiguous()
        w = w.permute(0, 2, 3, 1).contiguous()
    elif layout != "NCHW":
        raise ValueError(layout)
    return x, w, (b if bias else None)
