"""The oracle and the library's host-side planning, rebuilt with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only, on the CPU)
and run on many shapes; their results must equal the regular builds'.

- The oracle (oracle/conv_oracle.c) is built with gcc, without OpenMP, and
  driven by tests/sanitize/oracle_driver.c: padding-only windows, stride,
  dilation, both layouts, 1x1 and whole-input kernels, with and without bias.
  Its full and pointwise routines must agree, and y and D must equal the
  regular oracle's bit for bit (the same loops in the same order).
- The planner (conv_api.cpp, with the stem kernel's planner from
  patch_conv.hip) is built with hipcc for the host side under the
  sanitizers, every kernel launcher replaced by a stub that is never reached
  (tests/sanitize/igemm_stubs.cpp), and driven by
  tests/sanitize/planner_driver.cpp: workspace queries, rejected calls,
  output sizes and im2col bytes for thousands of seeded shapes over every
  layout, dtype, algorithm and forced main loop, including invalid and
  overflowing sizes.  Every answer must equal the regular library's.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import convolution_lowering_amd as cl
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "convolution_lowering_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-side sanitizers only; any report aborts the run
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...: rc {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def oracle_exe(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("san_oracle")
    exe = str(d / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "conv_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    return exe


@pytest.fixture(scope="module")
def planner_exe(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("san_planner")
    srcs = [os.path.join(CSRC, "conv_api.cpp"), os.path.join(CSRC, "patch_conv.hip"),
            os.path.join(SAN, "igemm_stubs.cpp"), os.path.join(SAN, "planner_driver.cpp")]
    objs, procs = [], []
    for s in srcs:
        o = str(d / (os.path.basename(s) + ".o"))
        objs.append(o)
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN_HOST + ["-c", s, "-o", o]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for cmd, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"{cmd[-1]}: {err[-3000:]}"
    exe = str(d / "planner_driver")
    _run([HIPCC, "--offload-arch=gfx950"] + SAN_HOST + objs + ["-o", exe])
    return exe


ORACLE_CASES = [
    # N, C, H, W, Co, KH, KW, s, p, d, layout, bias
    (2, 3, 7, 9, 4, 3, 3, 1, 1, 1, 0, True),
    (1, 2, 5, 5, 3, 3, 3, 2, 2, 2, 1, True),
    (2, 1, 4, 6, 2, 2, 3, 1, 4, 1, 0, False),   # windows that lie wholly in the padding
    (3, 5, 6, 6, 7, 1, 1, 1, 0, 1, 1, True),    # 1x1
    (2, 4, 5, 4, 6, 5, 4, 1, 0, 1, 0, True),    # whole-input kernel
    (1, 3, 11, 8, 5, 5, 3, 3, 3, 2, 1, False),
    (2, 6, 9, 10, 3, 7, 7, 2, 3, 1, 0, True),
]


@pytest.mark.parametrize("case", ORACLE_CASES, ids=[str(i) for i in range(len(ORACLE_CASES))])
def test_oracle_under_sanitizers(oracle_exe, tmp_path, case):
    N, C, H, W, Co, KH, KW, s, p, d, layout, has_b = case
    rng = np.random.default_rng(7 + sum(case[:10]))
    xs = (N, C, H, W) if layout == 0 else (N, H, W, C)
    ws = (Co, C, KH, KW) if layout == 0 else (Co, KH, KW, C)
    x, w = rng.standard_normal(xs), rng.standard_normal(ws)
    b = rng.standard_normal(Co) if has_b else None
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(fin, "wb") as f:
        np.array([N, C, H, W, Co, KH, KW, s, p, d, layout, int(has_b)], np.int32).tofile(f)
        x.tofile(f)
        w.tofile(f)
        if has_b:
            b.tofile(f)
    _run([oracle_exe, fin, fout], env=ENV)
    y_ref, dn_ref = oracle.conv2d(x, w, b, s, p, d, layout)
    got = np.fromfile(fout, np.float64)
    assert got.size == 2 * y_ref.size
    assert np.array_equal(got[:y_ref.size].reshape(y_ref.shape), y_ref)
    assert np.array_equal(got[y_ref.size:].reshape(y_ref.shape), dn_ref)


def _queries(n=4000, seed=11):
    rng = np.random.default_rng(seed)
    from convolution_lowering_amd.workloads import LAYERS
    q = []
    for L in LAYERS.values():
        for layout in (0, 1):
            for dt in range(4):
                for algo in range(8):
                    q.append((L.N, L.C, L.H, L.W, L.Co, L.KH, L.KW, L.stride, L.pad, L.dilation, layout, dt, algo, 0))
    pick = lambda *v: int(rng.choice(v))
    for _ in range(n):
        H = pick(1, 2, 7, 14, 28, 56, 97, 112, 224, 300)
        W = pick(1, 3, 8, 14, 20, 56, 83, 112, 224, 301)
        k = pick(1, 1, 3, 3, 5, 7)
        KH, KW = (H, W) if rng.random() < 0.05 else (k, pick(k, 1, 3))
        q.append((pick(1, 2, 3, 16, 64, 128, 300), pick(1, 3, 4, 8, 32, 37, 64, 96, 256, 512, 1024),
                  H, W, pick(1, 40, 61, 64, 100, 128, 256, 512, 1000), KH, KW, pick(1, 1, 2, 3), pick(0, 0, 1, 2, 4),
                  pick(1, 1, 2, 3), pick(0, 1), pick(0, 1, 2, 3), int(rng.integers(0, 8)),
                  pick(0, 0, 0, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15)))
    # invalid and overflowing sizes
    for v in (0, -1, 1 << 20, (1 << 31) - 1):
        q.append((v, 64, 56, 56, 128, 3, 3, 1, 1, 1, 0, 1, 0, 0))
        q.append((2, v, 56, 56, 128, 3, 3, 1, 1, 1, 1, 1, 0, 0))
        q.append((2, 64, v, v, 128, 3, 3, 1, 1, 1, 0, 1, 6, 0))
        q.append((2, 64, 56, 56, v, 3, 3, 1, 1, 1, 1, 0, 3, 0))
        q.append((2, 64, 56, 56, 128, v, v, 1, 1, 1, 0, 2, 1, 0))
        q.append((2, 64, 56, 56, 128, 3, 3, v, v, v, 1, 1, 2, 0))
    # (Enum arguments outside their enumerators are refused as well, which
    # the regular build's boundary tests check; a C++ driver cannot pass
    # them without itself loading an invalid enum value.)
    return q


def _regular(q):
    import ctypes
    lib = cl.lib()
    out = []
    for (N, C, H, W, Co, KH, KW, s, p, d, layout, dt, algo, ml) in q:
        fst = lib.conv2d_force_main_loop(ml)
        ws = ctypes.c_size_t(0)
        st = lib.conv2d_fwd_workspace_size(N, C, H, W, Co, KH, KW, s, p, d, layout, dt, algo, ctypes.byref(ws))
        fw = lib.conv2d_fwd(None, None, None, None, N, C, H, W, Co, KH, KW, s, p, d, layout, dt, None, None, 0, algo)
        ho, wo = ctypes.c_int(-1), ctypes.c_int(-1)
        os_ = lib.conv2d_output_size(H, W, KH, KW, s, p, d, ctypes.byref(ho), ctypes.byref(wo))
        ib = ctypes.c_size_t(0)
        is_ = lib.conv2d_im2col_bytes(N, C, H, W, KH, KW, s, p, d, dt, ctypes.byref(ib))
        lib.conv2d_force_main_loop(0)
        out.append(f"{fst} {st} {ws.value} {fw} {os_} {ho.value} {wo.value} {is_} {ib.value}")
    return out


def test_planner_under_sanitizers(planner_exe):
    q = _queries()
    text = "\n".join(" ".join(str(v) for v in row) for row in q) + "\n"
    env = dict(ENV, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0")  # the HIP runtime's own allocations live on
    r = _run([planner_exe], input=text, env=env, timeout=600)
    got = [" ".join(line.split()[:9]) for line in r.stdout.splitlines()]
    want = _regular(q)
    assert len(got) == len(want) == len(q)
    bad = [(q[i], got[i], want[i]) for i in range(len(q)) if got[i] != want[i]]
    assert not bad, f"{len(bad)} answers differ, first: {bad[:3]}"
    # the queries cover plans that need workspace and plans that are refused
    st = [int(g.split()[1]) for g in got]
    assert st.count(0) > 1000 and st.count(1) > 20 and st.count(2) > 100
