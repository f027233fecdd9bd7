"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
hand-worked cases, closed forms, a brute-force count, textbook identities
(1x1 convolution == matrix product, whole-input kernel == dense layer),
torch's own fp64 conv2d, and the unfold + matmul route of "Unifying
Convolutions and GEMM", section 5.
"""
import os
import re

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_case(path):
    vals = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            vals[key.strip()] = rest.strip()
    dims = {k: int(v) for k, v in re.findall(r"(\w+)=(-?\d+)", vals["shape"])}
    geo = {k: int(v) for k, v in re.findall(r"(\w+)=(-?\d+)", vals["geometry"])}

    def arr(s):
        return None if s == "none" else np.array([float(t) for t in s.split()])

    x = arr(vals["x"]).reshape(dims["N"], dims["C"], dims["H"], dims["W"])
    w = arr(vals["w"]).reshape(dims["Co"], dims["C"], dims["KH"], dims["KW"])
    b = arr(vals["bias"])
    y = arr(vals["y"])
    return dims, geo, x, w, b, y


CASES = sorted(f for f in os.listdir(GOLDEN) if f.startswith("case_"))


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("layout", [oracle.NCHW, oracle.NHWC])
def test_hand_cases(case, layout):
    dims, geo, x, w, b, y_exp = _parse_case(os.path.join(GOLDEN, case))
    if layout == oracle.NHWC:
        x = x.transpose(0, 2, 3, 1)
        w = w.transpose(0, 2, 3, 1)
    y, dn = oracle.conv2d(x, w, b, geo["stride"], geo["pad"], geo["dilation"], layout)
    if layout == oracle.NHWC:
        y, dn = y.transpose(0, 3, 1, 2), dn.transpose(0, 3, 1, 2)
    assert np.array_equal(y.reshape(-1), y_exp), (case, y.reshape(-1), y_exp)
    assert np.all(dn >= np.abs(y) - 1e-12)


def test_hand_case_rejects_a_flipped_kernel():
    """A planted mistake (a true convolution, i.e. flipped kernel) fails case A."""
    dims, geo, x, w, b, y_exp = _parse_case(os.path.join(GOLDEN, "case_A_no_flip.txt"))
    y_flipped = oracle.conv2d(x, w[:, :, ::-1, ::-1], b, want_norm=False)
    assert not np.array_equal(y_flipped.reshape(-1), y_exp)
    assert y_flipped.reshape(-1)[0] == 23.0


def _brute_force_placements(n_in, k, s, p, d):
    """Count window positions whose every tap lies in the padded extent."""
    count, start = 0, 0
    while start + (k - 1) * d <= n_in + 2 * p - 1:
        count += 1
        start += s
    return count


def test_out_size_against_brute_force_count():
    lib_calls = 0
    for n_in in range(1, 15):
        for k in range(1, 8):
            for s in range(1, 4):
                for p in range(0, 4):
                    for d in range(1, 4):
                        exp = _brute_force_placements(n_in, k, s, p, d)
                        assert oracle.out_size(n_in, k, s, p, d) == exp
                        assert oracle._load().oracle_out_size(n_in, k, s, p, d) == exp
                        lib_calls += 1
    assert lib_calls > 1000


@pytest.mark.parametrize("H,K,s,p,d,exp", [
    (224, 7, 2, 3, 1, 112),   # ResNet-50 stem
    (56, 3, 2, 1, 1, 28),     # 3x3 s2 with pad 1
    (56, 3, 2, 0, 1, 27),     # ... and with pad 0
    (97, 5, 2, 4, 2, 49),     # generality sweep, H
    (83, 5, 2, 4, 2, 42),     # generality sweep, W
    (7, 7, 1, 0, 1, 1),       # kernel == whole input
    (56, 3, 1, 1, 1, 56),     # the blog's verification layer
])
def test_out_size_named_layers(H, K, s, p, d, exp):
    assert oracle.out_size(H, K, s, p, d) == exp == _brute_force_placements(H, K, s, p, d)


def test_1x1_stride1_is_a_plain_matrix_product():
    """The Indirect Convolution Algorithm (abstract): a 1x1 convolution is a GEMM."""
    rng = np.random.default_rng(11)
    N, C, H, W, Co = 3, 13, 5, 7, 9
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C, 1, 1))
    b = rng.standard_normal(Co)
    y = oracle.conv2d(x, w, b, want_norm=False)
    for n in range(N):
        ref = w[:, :, 0, 0] @ x[n].reshape(C, H * W) + b[:, None]
        np.testing.assert_allclose(y[n].reshape(Co, H * W), ref, rtol=1e-13, atol=1e-13)


def test_whole_input_kernel_is_a_dense_layer():
    """"Unifying Convolutions and GEMM", section 4: K_H = H, K_W = W gives a
    1x1 output equal to the dense layer x_flat @ W_flat^T + b."""
    rng = np.random.default_rng(12)
    N, C, H, W, Co = 4, 6, 5, 4, 7
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C, H, W))
    b = rng.standard_normal(Co)
    y = oracle.conv2d(x, w, b, want_norm=False)
    assert y.shape == (N, Co, 1, 1)
    ref = x.reshape(N, -1) @ w.reshape(Co, -1).T + b
    np.testing.assert_allclose(y[:, :, 0, 0], ref, rtol=1e-13, atol=1e-13)


def test_nhwc_equals_permuted_nchw_bitwise():
    rng = np.random.default_rng(13)
    N, C, H, W, Co, K = 2, 5, 9, 8, 4, 3
    x = rng.integers(-3, 4, (N, C, H, W)).astype(np.float64)
    w = rng.integers(-3, 4, (Co, C, K, K)).astype(np.float64)
    b = rng.integers(-3, 4, Co).astype(np.float64)
    y1, d1 = oracle.conv2d(x, w, b, 2, 1, 2, oracle.NCHW)
    y2, d2 = oracle.conv2d(x.transpose(0, 2, 3, 1), w.transpose(0, 2, 3, 1), b, 2, 1, 2, oracle.NHWC)
    assert np.array_equal(y1, y2.transpose(0, 3, 1, 2))
    assert np.array_equal(d1, d2.transpose(0, 3, 1, 2))


def _sweep(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        H, W = rng.integers(1, 13, 2)
        KH, KW = rng.integers(1, 6, 2)
        s, d = rng.integers(1, 4, 2)
        p = int(rng.integers(0, 5))
        if oracle.out_size(H, KH, s, p, d) <= 0 or oracle.out_size(W, KW, s, p, d) <= 0:
            continue
        N, C, Co = rng.integers(1, 4), rng.integers(1, 6), rng.integers(1, 6)
        out.append(tuple(int(v) for v in (N, C, H, W, Co, KH, KW, s, p, d)))
    return out


@pytest.mark.parametrize("shape", _sweep(21, 60))
def test_against_torch_conv2d_fp64(shape):
    """The routine the blog's section 5 verifies against (F.conv2d), in fp64."""
    N, C, H, W, Co, KH, KW, s, p, d = shape
    g = torch.Generator().manual_seed(hash(shape) & 0xFFFF)
    x = torch.randn(N, C, H, W, generator=g, dtype=torch.float64)
    w = torch.randn(Co, C, KH, KW, generator=g, dtype=torch.float64)
    b = torch.randn(Co, generator=g, dtype=torch.float64)
    ref = F.conv2d(x, w, b, stride=s, padding=p, dilation=d).numpy()
    y, dn = oracle.conv2d(x.numpy(), w.numpy(), b.numpy(), s, p, d)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # the normaliser is the same convolution taken over absolute values
    dref = F.conv2d(x.abs(), w.abs(), b.abs(), stride=s, padding=p, dilation=d).numpy()
    np.testing.assert_allclose(dn, dref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", _sweep(22, 20))
def test_against_unfold_matmul_route(shape):
    """The lowering of "Unifying Convolutions and GEMM", section 5: unfold,
    transpose, W.view(C_out, -1), matmul, + bias, reshape -- with dilation."""
    N, C, H, W, Co, KH, KW, s, p, d = shape
    g = torch.Generator().manual_seed(7 + (hash(shape) & 0xFFFF))
    x = torch.randn(N, C, H, W, generator=g, dtype=torch.float64)
    w = torch.randn(Co, C, KH, KW, generator=g, dtype=torch.float64)
    b = torch.randn(Co, generator=g, dtype=torch.float64)
    Ho, Wo = oracle.out_size(H, KH, s, p, d), oracle.out_size(W, KW, s, p, d)
    cols = F.unfold(x, (KH, KW), dilation=d, padding=p, stride=s).transpose(1, 2)
    y_col = torch.matmul(cols, w.reshape(Co, -1).t()) + b
    ref = y_col.transpose(1, 2).reshape(N, Co, Ho, Wo).numpy()
    y = oracle.conv2d(x.numpy(), w.numpy(), b.numpy(), s, p, d, want_norm=False)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_integer_inputs_match_torch_exactly():
    g = torch.Generator().manual_seed(5)
    x = torch.randint(-3, 4, (2, 7, 11, 10), generator=g).double()
    w = torch.randint(-3, 4, (5, 7, 3, 3), generator=g).double()
    b = torch.randint(-3, 4, (5,), generator=g).double()
    ref = F.conv2d(x, w, b, stride=1, padding=1).numpy()
    y = oracle.conv2d(x.numpy(), w.numpy(), b.numpy(), 1, 1, 1, want_norm=False)
    assert np.array_equal(y, ref)


def test_points_equal_full_output():
    rng = np.random.default_rng(14)
    N, C, H, W, Co = 2, 4, 9, 7, 3
    x = rng.standard_normal((N, H, W, C))
    w = rng.standard_normal((Co, 3, 3, C))
    b = rng.standard_normal(Co)
    y, dn = oracle.conv2d(x, w, b, 2, 2, 1, oracle.NHWC)
    Ho, Wo = y.shape[1], y.shape[2]
    pts = np.array([(n, co, ho, wo) for n in range(N) for co in range(Co)
                    for ho in range(Ho) for wo in range(Wo)], np.int32)
    yp, dp = oracle.conv2d_points(x, w, b, pts, 2, 2, 1, oracle.NHWC)
    assert np.array_equal(yp, y[pts[:, 0], pts[:, 2], pts[:, 3], pts[:, 1]])
    assert np.array_equal(dp, dn[pts[:, 0], pts[:, 2], pts[:, 3], pts[:, 1]])


def test_no_bias_and_all_padding_windows():
    """A window entirely in the padding with no bias yields exactly 0 and D = 0."""
    x = np.ones((1, 1, 2, 2))
    w = np.ones((1, 1, 1, 1))
    y, dn = oracle.conv2d(x, w, None, 1, 2, 1)
    assert y.shape == (1, 1, 6, 6)
    assert y[0, 0, 0, 0] == 0.0 and dn[0, 0, 0, 0] == 0.0
    assert y[0, 0, 2, 2] == 1.0
