"""The generated one-pass forward+backward kernels run on the CPU.

The HIP source a plan generates is compiled for the host with a thin shim
(tests/emu/shim.h: one thread per lane, LDS as shared statics, shuffles and
wavefront syncs through a barrier), AddressSanitizer and
UndefinedBehaviorSanitizer, every buffer allocated at its exact size, and
launched over the same grid the library uses.  Checked: no access outside
any buffer, no undefined behaviour (shifts, signed overflow, misaligned or
null accesses, invalid loads), and the outputs against the oracle.  The case is the one whose FP64 form took a device memory fault on
the GPU (128-channel plan, SH computed from edge vectors, forces from the
per-unit SH-gradient partials): the FP64 one-pass kernel stays switched off
on the device; this shows that the code generated now stays in bounds for
those exact inputs, in both call forms the library issues, and computes the
oracle's values.  No GPU is used.
"""
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from clebsch_gordan_tensor_cg_amd import workloads as W
from tests.gpu_util import GraphArrays, rel_err

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang++"


def _edge_vectors(rng, E, dtype):
    v = rng.standard_normal((E, 3)) * 2.0
    return W.round_to(v, dtype) if dtype != "f64" else v


@pytest.fixture(scope="module")
def B():
    from clebsch_gordan_tensor_cg_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from clebsch_gordan_tensor_cg_amd import build
        build.build(verbose=False)
    return binding


def _grid(src_text):
    body = src_text[src_text.index("void cgtp_fb_body("):]
    units = int(re.search(r"const int unit = \(int\)\(blk % (\d+)\);", body).group(1))
    m = re.search(r"const long long n0 = \(blk / \d+\) \* (\d+) \+ lane / \d+;", body)
    ipw = int(m.group(1)) if m else 1
    spec = int(re.search(r"cgtp_fb_body<(\d+)>\(", src_text[src_text.index(") cgtp_fb_full("):]).group(1))
    return units, ipw, spec


@pytest.mark.skipif(not os.path.exists(CLANG), reason="host clang++ not found")
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_one_pass_kernel_emulated(B, tmp_path, dtype):
    a, b = "128x0e+128x1o", "1x0e+1x1o+1x2e+1x3o"
    c, paths = W.one_block_per_path(a, b, ["0e", "1o", "2e", "3o"])
    plan = B.Plan(a, b, c, paths, "uvu", dtype, no_load=True)
    prob = oracle.Problem(a, b, c, "uvu", paths)
    src_text = plan.source()
    units, ipw, spec = _grid(src_text)
    # the inputs of the GPU test of this case (128-channel plan, SH from vectors)
    rs = np.random.default_rng(162)
    n = 61
    s_, d_ = rs.integers(0, n, 700), rs.integers(0, n, 700)
    d_[d_ == 5] = 6
    order = np.lexsort((d_, s_))
    src, dst = s_[order].astype(np.int32), d_[order].astype(np.int32)
    G = GraphArrays(src, dst, n)
    rng = np.random.default_rng(172)
    x = W.normal(rng, (n, prob.dim1), dtype)
    w = W.normal(rng, (G.E, prob.weight_numel), dtype)
    g = W.normal(rng, (n, prob.dim3), dtype)
    vec = _edge_vectors(rng, G.E, dtype)
    f = np.float64 if dtype == "f64" else np.float32
    wr = lambda name, arr, t: np.ascontiguousarray(arr, dtype=t).tofile(str(tmp_path / name))
    wr("x.bin", x, f); wr("w.bin", w[G.perm], f); wr("g.bin", g, f); wr("vec.bin", vec, f)
    wr("src.bin", G.src_d, np.int32); wr("rp.bin", G.row_ptr, np.int32); wr("vperm.bin", G.perm, np.int32)
    (tmp_path / "kernel.inc").write_text(src_text)
    exe = tmp_path / "run_fb"
    cmd = [CLANG, "-std=c++20", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer",
           "-D__HIPCC_RTC__", f"-DREAL={'double' if dtype == 'f64' else 'float'}", "-I", str(tmp_path),
           "-I", os.path.join(HERE, "emu"), os.path.join(HERE, "emu", "run_fb.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)

    sh = oracle.spherical_harmonics(3, vec.astype(np.float64))
    ref = prob.conv_forward(x, sh, w, src, dst, n)
    gx, gy, gw = prob.conv_backward(x, sh, w, src, dst, g)
    tol = 1e-12 if dtype == "f64" else 1e-5
    parts = units > 1
    # the library's two calls of this test: every gradient (g_w, x-messages,
    # SH-gradient partials), then forces only (partials alone); the first
    # also through the kernel with those flags folded in
    full_flags = 1 | 2 | 4 | (64 if parts else 0)
    assert spec == full_flags
    for full, flags in ((1, full_flags), (0, full_flags), (0, 4 | (64 if parts else 0))):
        r = subprocess.run([str(exe), str(full), str(n), str(G.E), str(prob.dim1), str(prob.dim2), str(prob.dim3),
                            str(prob.weight_numel), str(units), str(ipw), str(flags), "1"],
                           cwd=tmp_path, capture_output=True, text=True, timeout=600,
                           env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1"))
        assert r.returncode == 0 and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, \
            r.stderr[-3000:]
        rd = lambda name, cnt: np.fromfile(str(tmp_path / name), dtype=f, count=cnt)
        out = rd("out_emu.bin", n * prob.dim3).reshape(n, prob.dim3)
        assert rel_err(out, ref) <= tol
        third = rd("third_emu.bin", -1).reshape(units if parts else 1, G.E, prob.dim2).sum(axis=0)
        assert rel_err(third, gy[G.perm]) <= tol, "SH gradient"
        if flags & 1:
            assert rel_err(rd("gw_emu.bin", -1).reshape(G.E, -1), gw[G.perm]) <= tol, "g_w"
        if flags & 2:
            m = rd("m_emu.bin", -1).reshape(G.E, prob.dim1).astype(np.float64)
            g_x = np.zeros((n, prob.dim1))
            np.add.at(g_x, G.src_d, m)
            assert rel_err(g_x, gx) <= tol, "g_x from the x-messages"
