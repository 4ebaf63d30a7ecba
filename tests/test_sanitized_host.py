"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU (no GPU is touched):

- the oracle built with gcc -fsanitize=address,undefined runs every one of
  its functions on small inputs, in a child process that preloads the
  sanitizer runtimes, and gives the same values as the plain build;
- the library built with host-only sanitizers (each -fsanitize= after
  -Xarch_host: the device code is not instrumented) plans the standard
  workloads without loading anything (code objects from the cache the build
  fills), answers the plan queries and dumps the plans, and rejects bad
  arguments of the execution calls before any launch.

Any report makes the child exit non-zero (halt_on_error, no recovery).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

ORACLE_RUN = r'''
import sys, numpy as np
sys.path.insert(0, %(root)r)
import oracle
from clebsch_gordan_tensor_cg_amd import workloads as W
rng = np.random.default_rng(5)
out = {}
for l1, l2, l3 in [(1, 1, 0), (2, 3, 4), (6, 6, 6), (3, 2, 1)]:
    out["cg%%d%%d%%d" %% (l1, l2, l3)] = oracle.real_cg(l1, l2, l3)
vec = rng.standard_normal((40, 3))
out["sh"] = oracle.spherical_harmonics(6, vec)
out["jac"] = oracle.sh_jacobian(3, vec)
a, b = "5x0e+3x1o+2x2e", "1x0e+1x1o+1x2e"
c, paths = W.one_block_per_path(a, b, ["0e", "1o", "2e"])
prob = oracle.Problem(a, b, c, "uvu", paths)
n, E = 9, 40
src = rng.integers(0, n, E); dst = rng.integers(0, n, E)
x = rng.standard_normal((n, prob.dim1)); y = rng.standard_normal((E, prob.dim2))
w = rng.standard_normal((E, prob.weight_numel)); g = rng.standard_normal((n, prob.dim3))
out["tp"] = prob.tp_forward(x[:7], y[:7], w[:7])
out["tpb"] = np.concatenate([v.ravel() for v in prob.tp_backward(x[:7], y[:7], w[:7], g[:7])])
out["conv"] = prob.conv_forward(x, y, w, src, dst, n)
out["bwd"] = np.concatenate([v.ravel() for v in prob.conv_backward(x, y, w, src, dst, g)])
out["dbl"] = np.concatenate([v.ravel() for v in prob.conv_double_backward(
    x, y, w, src, dst, g, rng.standard_normal(x.shape), rng.standard_normal(y.shape), rng.standard_normal(w.shape))
    if v is not None])
vec2 = rng.standard_normal((E, 3))
gsh = rng.standard_normal((E, 16))
out["forces"] = oracle.forces(3, n, src, dst, vec2, gsh)
out["cot"] = oracle.force_loss_cotangent(3, n, src, dst, vec2, rng.standard_normal((n, 3)))
perm, rp = oracle.csr(dst, n)
out["csr"] = np.concatenate([perm, rp]).astype(np.float64)
uvw_a, uvw_c = "4x0+3x1", "5x0+2x1"
pu = oracle.Problem(uvw_a, "1x0+1x1", uvw_c, "uvw", None, True)
wu = rng.standard_normal((1, pu.weight_numel))
out["uvw"] = pu.conv_forward(rng.standard_normal((n, pu.dim1)), rng.standard_normal((E, pu.dim2)), wu, src, dst, n)
q = rng.standard_normal((n, 2, 4)); k = rng.standard_normal((n, 2, 4)); v = rng.standard_normal((n, 2, 4))
out["attn"] = oracle.sparse_attention(q, k, v, src, dst, n, 0.5)
np.savez(%(dest)r, **out)
'''

LIB_RUN = r'''
import ctypes, os, sys
sys.path.insert(0, %(root)r)
from clebsch_gordan_tensor_cg_amd import workloads as W
L = ctypes.CDLL(%(lib)r)
vp = ctypes.c_void_p
L.cgtp_plan.argtypes = [ctypes.c_char_p] * 3 + [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                        ctypes.c_uint32, vp]
L.cgtp_last_error.restype = ctypes.c_char_p
DT = {"f32": 0, "f64": 1, "bf16": 2}
class P(ctypes.Structure):
    _fields_ = [("i1", ctypes.c_int32), ("i2", ctypes.c_int32), ("i3", ctypes.c_int32)]
class D(ctypes.Structure):
    _fields_ = [("d1", ctypes.c_int64), ("d2", ctypes.c_int64), ("d3", ctypes.c_int64), ("wn", ctypes.c_int64),
                ("np", ctypes.c_int32), ("lmax", ctypes.c_int32), ("nk", ctypes.c_int32), ("cached", ctypes.c_int32)]
for name in ("c1", "c2", "c3", "c5"):
    c = W.config(name)
    paths = (P * len(c.paths))(*[P(*t) for t in c.paths]) if c.paths else None
    h = vp()
    flags = 2 | (1 if c.shared_weights else 0)      # CGTP_PLAN_NO_LOAD (| CGTP_SHARED_WEIGHTS)
    rc = L.cgtp_plan(c.irreps_in1.encode(), c.irreps_in2.encode(), c.irreps_out.encode(), paths,
                     len(c.paths) if c.paths else 0, 1 if c.mode == "uvw" else 0, DT[c.dtype], flags, ctypes.byref(h))
    assert rc == 0, (name, L.cgtp_last_error())
    d = D()
    assert L.cgtp_plan_info(h, ctypes.byref(d)) == 0, name
    buf = (P * 64)()
    assert L.cgtp_plan_paths(h, buf, 64) == 0 or d.np > 64
    n = ctypes.c_int64()
    assert L.cgtp_plan_source(h, None, ctypes.c_int64(0), ctypes.byref(n)) == 0 and n.value > 0
    src = ctypes.create_string_buffer(n.value + 1)
    assert L.cgtp_plan_source(h, src, ctypes.c_int64(n.value + 1), ctypes.byref(n)) == 0
    R = (ctypes.c_double * (13 * 13 * 13))()
    for p_ in range(d.np):
        assert L.cgtp_plan_coupling(h, p_, R, ctypes.c_int64(13 * 13 * 13)) == 0
    ws = ctypes.c_size_t()
    assert L.cgtp_workspace_bytes(h, ctypes.c_int64(100), ctypes.c_int64(1000), ctypes.byref(ws)) == 0
    # execution calls on a plan that loaded nothing: refused before any launch
    assert L.cgtp_forward(h, None, None, None, ctypes.c_int64(1), None, None, ctypes.c_size_t(0), None) != 0
    L.cgtp_plan_destroy(h)
# bad plans and helper arguments: refused on the host
h = vp()
assert L.cgtp_plan(b"2x0e+", b"1x0e", b"2x0e", None, 0, 0, 0, 2, ctypes.byref(h)) != 0
assert L.cgtp_plan(b"1x7e", b"1x0e", b"1x7e", None, 0, 0, 0, 2, ctypes.byref(h)) != 0
buf = (ctypes.c_int32 * 16)()
assert L.cgtp_build_csr_transpose_canonical(buf, buf, ctypes.c_int64(-1), ctypes.c_int64(3), buf, buf, None) != 0
assert L.cgtp_stream_probe(3, buf, buf, ctypes.c_size_t(16), None) != 0
print("library host code clean")
'''


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not found")
    so = str(tmp_path / "libcgtp_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "cgtp_oracle.c"), "-o", so, "-lm"], check=True, timeout=300)
    results = {}
    for tag, extra in (("san", {"CGTP_ORACLE_LIB": so, "LD_PRELOAD": f"{asan}:{ubsan}"}), ("plain", {})):
        dest = str(tmp_path / f"{tag}.npz")
        env = dict(os.environ, OMP_NUM_THREADS="2", **SAN_ENV, **extra)
        r = subprocess.run([sys.executable, "-c", ORACLE_RUN % {"root": ROOT, "dest": dest}], env=env,
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0 and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, \
            r.stderr[-4000:]
        results[tag] = dest
    import numpy as np
    a, b = np.load(results["san"]), np.load(results["plain"])
    assert sorted(a.files) == sorted(b.files)
    for k in a.files:
        np.testing.assert_allclose(a[k], b[k], rtol=1e-12, atol=1e-12, err_msg=k)


def test_library_host_code_under_sanitizers(tmp_path):
    from clebsch_gordan_tensor_cg_amd import build
    import glob
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not found")
    lib = str(tmp_path / "libcgtp_san.so")
    build.build(verbose=False, out=lib, build_dir=str(tmp_path / "obj"),
                extra=["-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                       "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"])
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=rt[-1],
               CGTP_CACHE_DIR=os.path.join(ROOT, "clebsch_gordan_tensor_cg_amd", "_kcache"), CGTP_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", LIB_RUN % {"root": ROOT, "lib": lib}], env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, \
        (r.stdout[-2000:], r.stderr[-4000:])
    assert "library host code clean" in r.stdout
    assert r.stderr.count("cgtp plan:") == 4
